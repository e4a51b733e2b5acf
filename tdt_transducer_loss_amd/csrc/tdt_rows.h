// Streaming passes over the token-logit rows of the joint output:
//   row partials — per row segment, the log-sum-exp partial of the V token logits
//                  (the per-node log-softmax of the page "tdt-loss: add TDT loss
//                  kernel", comment "What's in it"), plus the blank and label logits;
//   gradient     — d loss / d token logit for every column of every node, zeros at
//                  padded nodes, written in the logits' dtype (the fused gradient
//                  kernel of the same comment).
//
// A row of V elements is covered by the 16-byte aligned chunks that overlap it (an
// aligned chunk holding a byte of the row never leaves that row's page); the first and
// last chunk are read element by element and written slot by slot.  Each pass splits a
// row into segments of up to NCH windows of 64 chunks (NCH <= 8 for the row statistics,
// <= 4 for the gradient pass: pick_segments), one 64-lane wave per segment, so that a
// wave keeps at most 8 chunks (32 VGPRs) of raw data in flight and many waves fit on each
// SIMD.
#pragma once

#include "tdt_common.h"

namespace tdt {

constexpr int kWavesPerBlock = 4;   // 256-thread work-groups
// Grid of the persistent row-statistics pass: about two (node, segment) tasks per wave,
// at most 12288 blocks (48K waves).  Measured at B4 T200 U40 V8193 bf16 (98,400 tasks):
// 4096 blocks 109 us, 12288 (two tasks per wave) 102 us, 16384 (one or two) 118 us,
// 32768 (one) 109 us.
constexpr int kRowStatBlocks = 12288;
constexpr int kRowStatTasksPerWave = 2;
static_assert(kRowStatBlocks % 8 == 0, "whole rounds of the eight XCDs");

template <typename TI>
__device__ __forceinline__ uint4 neg_inf_chunk() {
  const uint32_t w = TI::kEpc == 4 ? TI::kNegInf : (TI::kNegInf | (TI::kNegInf << 16));
  return make_uint4(w, w, w, w);
}

// Running maximum of the raw chunk words, in a form that shares no arithmetic with the
// float decode of the exp pass (so the compiler keeps only the raw words alive).
//   fp32: float max;  fp16: packed half max;  bf16: packed signed-int16 max of the raw
//   words, exact when the lane holds a non-negative value (non-negative bf16 values order
//   like their bit patterns); a segment with no non-negative value takes an exact second
//   pass over order-preserving keys (negative values get their magnitude bits flipped).
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));

template <typename TI>
struct MaxAcc;

template <>
struct MaxAcc<F32> {
  float m = -__builtin_inff();
  __device__ __forceinline__ void add(uint32_t w) { m = fmaxf(m, __uint_as_float(w)); }
  __device__ __forceinline__ float value() const { return m; }
};

template <>
struct MaxAcc<F16> {
  h16x2 m = {(_Float16)-__builtin_inff(), (_Float16)-__builtin_inff()};
  __device__ __forceinline__ void add(uint32_t w) {
    m = __builtin_elementwise_max(m, __builtin_bit_cast(h16x2, w));
  }
  __device__ __forceinline__ float value() const { return fmaxf((float)m.x, (float)m.y); }
};

template <>
struct MaxAcc<BF16> {
  s16x2 m = {(short)-32768, (short)-32768};
  __device__ __forceinline__ void add(uint32_t w) { m = __builtin_elementwise_max(m, __builtin_bit_cast(s16x2, w)); }
  // the lane's maximum when it is non-negative, else -inf
  __device__ __forceinline__ float value() const {
    const short k = m.x > m.y ? m.x : m.y;
    return k >= 0 ? __uint_as_float(((uint32_t)(uint16_t)k) << 16) : -__builtin_inff();
  }
};

// exact bf16 maximum of raw words through order-preserving keys
struct KeyMaxBF16 {
  s16x2 m = {(short)-32768, (short)-32768};
  __device__ __forceinline__ void add(uint32_t w) {
    const s16x2 x = __builtin_bit_cast(s16x2, w);
    m = __builtin_elementwise_max(m, x ^ ((x >> (short)15) & (short)0x7fff));
  }
  __device__ __forceinline__ float value() const {
    const short k = m.x > m.y ? m.x : m.y;
    const short x = k ^ ((k >> 15) & 0x7fff);
    return __uint_as_float(((uint32_t)(uint16_t)x) << 16);
  }
};

// Row geometry shared by the two passes.
struct RowCover {
  const uint4* base;  // first 16-byte chunk overlapping the row
  int head;           // elements of chunk 0 before the row starts
  int nch;            // chunks overlapping the row
};

template <typename TI>
__device__ __forceinline__ RowCover row_cover(const void* row, int V) {
  constexpr int EPC = TI::kEpc;
  const uintptr_t a = (uintptr_t)row;
  RowCover rc;
  rc.base = (const uint4*)(a & ~(uintptr_t)15);
  rc.head = (int)((a & 15) / sizeof(typename TI::T));
  rc.nch = (rc.head + V + EPC - 1) / EPC;
  return rc;
}

// Exponent (base 2) of one element relative to the segment's shift:
//   fp32:   (x - c) log2e with c the segment maximum (exact difference, one rounding);
//   16-bit: fma(x, log2e, -c) with c = round(maximum * log2e) (one instruction; c is
//           stored, so the sum and every later use of it agree on the same shift).
template <typename TI>
__device__ __forceinline__ float expo(float x, float c) {
  if constexpr (TI::kEpc == 4) return (x - c) * kLog2e;
  else return __builtin_fmaf(x, kLog2e, -c);
}

// Partial log-sum-exp of one row segment.  Writes, per (node, segment):
//   part[2*seg] = c, part[2*seg + 1] = sum 2^expo(h, c)
// (floats, in a [positions][2*nseg] array), and the blank / label logits into stat.
// A segment is NCH windows of 64 16-byte chunks, one chunk per lane per window; windows
// that hold no chunk of the row are skipped.  The first and the last chunk of the row
// (which may hold elements of other rows) are left out of the chunk windows and read
// element by element, one element per lane, so the windows need no per-element masks.
template <typename TI, int NCH>
__global__ __launch_bounds__(256) void k_row_partial(const Params p) {
  constexpr int EPC = TI::kEpc;
  using ET = typename TI::T;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (blockIdx.x == 0)  // the flags the node-weight kernel of this call sets
    for (int i = threadIdx.x; i < p.B; i += blockDim.x) p.xflag[i] = 0;
  // persistent: a fixed grid of waves walks the (node, segment) space of the padded
  // [B, Tmax, U1max] rows in memory order, skipping nodes outside their utterance in a
  // few instructions (ragged batches leave most of the padded space empty); the host
  // keeps this space below 2^31
  const uint32_t nseg = (uint32_t)p.nseg;
  const uint32_t per = (uint32_t)p.Tmax * (uint32_t)p.U1max;
  const uint32_t total = (uint32_t)p.B * per * nseg;
  const uint32_t stride = gridDim.x * kWavesPerBlock;
  for (uint32_t g = xcd_block(blockIdx.x, gridDim.x) * kWavesPerBlock + wv; g < total; g += stride) {
    const uint32_t node = fdiv(g, p.fd_nseg);
    const int seg = (int)(g - node * nseg);
    const uint32_t b = fdiv(node, p.fd_tu1);
    const uint32_t nrem = node - b * per;
    const int t = (int)fdiv(nrem, p.fd_u1);
    const int u = (int)(nrem - (uint32_t)t * (uint32_t)p.U1max);
    const int64_t T64 = p.Tlen[b], U64 = p.Ulen[b];
    if (!utt_dims_ok(p, T64, U64)) continue;
    const int T = (int)T64, U = (int)U64;
    if (t >= T || u > U) continue;
    // its position in the diagonal-major workspace layout
    const int64_t pos = node_pos(p, (int)b, t, u);

    const int V = p.V;
    const ET* row = (const ET*)p.tok + ((int64_t)b * p.ts0 + (int64_t)t * p.ts1 + (int64_t)u * p.ts2);
    const RowCover rc = row_cover<TI>(row, V);
    const int nch = rc.nch;
    const int c0 = seg * 64 * NCH;
    const int nwin = (nch - c0 + 63) >> 6;  // windows of this segment holding chunks (may exceed NCH)
    // range-checked loads: chunks at or past the end of the row read as zero bits (and
    // are masked below)
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)rc.base, (short)0, nch * 16, 0x00020000);
    uint4 v[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      if (j < nwin) {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (c0 + lane + 64 * j) * 16, 0, 0);
        v[j] = make_uint4(x.x, x.y, x.z, x.w);
      }
    }
    // the first and the last chunk of the row, element by element: elements [0, eh) in
    // the segment holding chunk 0, elements [V - et, V) in the segment holding chunk nch-1
    const int eh = c0 == 0 ? min(V, EPC - rc.head) : 0;
    const bool tail_here = nch > 1 && nch - 1 >= c0 && nch - 1 < c0 + 64 * NCH;
    const int et = tail_here ? V - ((nch - 1) * EPC - rc.head) : 0;
    float xe = -__builtin_inff();
    if (lane < eh) xe = TI::load(row, lane);
    else if (lane - eh < et) xe = TI::load(row, V - et + (lane - eh));
    // the blank and label logits, by the segment that holds their chunk
    const int seg_span = 64 * NCH;
    float* rs = (float*)(p.stat + pos);
    if (lane == 0) {
      if ((rc.head + p.blank) / EPC / seg_span == seg) rs[0] = TI::load(row, p.blank);
      int y = -1;
      if (u < U) {
        const int64_t yy = p.labels[(int64_t)b * p.lab_stride + u];
        if (yy >= 0 && yy < V) y = (int)yy;
      }
      if (y >= 0 ? (rc.head + y) / EPC / seg_span == seg : seg == 0)
        rs[1] = y >= 0 ? TI::load(row, y) : -__builtin_inff();
    }
    // chunk 0, chunk nch-1 and chunks past the row hold no element for the windows
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int cw = c0 + 64 * j;
      if (j < nwin && (cw == 0 || cw + 63 >= nch - 1)) {
        const int c = cw + lane;
        if (c == 0 || c >= nch - 1) v[j] = neg_inf_chunk<TI>();
      }
    }
    MaxAcc<TI> mx;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      if (j < nwin) {
        mx.add(v[j].x);
        mx.add(v[j].y);
        mx.add(v[j].z);
        mx.add(v[j].w);
      }
    }
    float mw = wave_max_dpp(fmaxf(mx.value(), xe));
    if constexpr (__is_same(TI, BF16)) {
      if (!(mw >= 0.f)) {  // no non-negative value in the segment: exact maximum from keys
        KeyMaxBF16 km;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          if (j < nwin) {
            km.add(v[j].x);
            km.add(v[j].y);
            km.add(v[j].z);
            km.add(v[j].w);
          }
        }
        mw = wave_max_dpp(fmaxf(km.value(), xe));
      }
    }
    // the shift: the maximum itself (fp32) or maximum * log2e rounded to float (16-bit)
    const float c = EPC == 4 ? mw : mw * kLog2e;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      if (j < nwin) {
#pragma unroll
        for (int s = 0; s < EPC; ++s) {
          const float e2 = __builtin_amdgcn_exp2f(expo<TI>(TI::get(v[j], s), c));
          if ((s & 3) == 0) a0 += e2;
          else if ((s & 3) == 1) a1 += e2;
          else if ((s & 3) == 2) a2 += e2;
          else a3 += e2;
        }
      }
    }
    float acc = ((a0 + a1) + (a2 + a3)) + __builtin_amdgcn_exp2f(expo<TI>(xe, c));
    const bool empty = !(mw > -__builtin_inff());  // every slot masked: an empty segment
    if (empty) acc = 0.f;
    double S = wave_sum_dpp((double)acc);
    // 16-bit logits beyond about 2.3e38 in magnitude leave no float shift: NaN partial
    if (!empty && !(__builtin_fabsf(c) < __builtin_inff())) S = __builtin_nan("");
    if (lane == 0) {
      float* part = p.part + (pos * nseg + seg) * 2;
      part[0] = empty ? -__builtin_inff() : c;
      part[1] = (float)S;
    }
  }
}

// Row statistics for short segments (at most 4 windows): the same task as
// k_row_partial, split into its loads (row_task_load) and its reductions
// (row_task_finish), so that a wave issues the loads of both of its tasks before reducing
// either.  With longer segments the second task's registers cost more occupancy than the
// overlap gains (B4 T200 U40 V8193 bf16, 6-window segments: 107 vs 104 us; the ragged fp16
// batch, 3-window segments: 200 vs 210 us; B2 T1000 U1500 V1025 bf16: 2.17 vs 2.38 ms).
template <typename TI, int NCH>
struct RowTask {
  bool ok;  // a node of its utterance's lattice (wave-uniform)
  int seg, c0, nwin, nch;
  int64_t pos;      // workspace position of the node
  uint4 v[NCH];
  float xe;
};

template <typename TI, int NCH>
__device__ __forceinline__ void row_task_load(const Params& p, uint32_t g, uint32_t total, int lane,
                                              RowTask<TI, NCH>& tk) {
  constexpr int EPC = TI::kEpc;
  using ET = typename TI::T;
  tk.ok = false;
  if (g >= total) return;
  const uint32_t nseg = (uint32_t)p.nseg;
  const uint32_t per = (uint32_t)p.Tmax * (uint32_t)p.U1max;
  const uint32_t node = fdiv(g, p.fd_nseg);
  const int seg = (int)(g - node * nseg);
  const uint32_t b = fdiv(node, p.fd_tu1);
  const uint32_t nrem = node - b * per;
  const int t = (int)fdiv(nrem, p.fd_u1);
  const int u = (int)(nrem - (uint32_t)t * (uint32_t)p.U1max);
  const int64_t T64 = p.Tlen[b], U64 = p.Ulen[b];
  if (!utt_dims_ok(p, T64, U64)) return;
  const int T = (int)T64, U = (int)U64;
  if (t >= T || u > U) return;
  tk.ok = true;
  tk.seg = seg;
  tk.pos = node_pos(p, (int)b, t, u);
  const int V = p.V;
  const ET* row = (const ET*)p.tok + ((int64_t)b * p.ts0 + (int64_t)t * p.ts1 + (int64_t)u * p.ts2);
  const RowCover rc = row_cover<TI>(row, V);
  const int nch = rc.nch;
  const int c0 = seg * 64 * NCH;
  const int nwin = (nch - c0 + 63) >> 6;
  tk.nch = nch;
  tk.c0 = c0;
  tk.nwin = nwin;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)rc.base, (short)0, nch * 16, 0x00020000);
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    if (j < nwin) {
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (c0 + lane + 64 * j) * 16, 0, 0);
      tk.v[j] = make_uint4(x.x, x.y, x.z, x.w);
    }
  }
  const int eh = c0 == 0 ? min(V, EPC - rc.head) : 0;
  const bool tail_here = nch > 1 && nch - 1 >= c0 && nch - 1 < c0 + 64 * NCH;
  const int et = tail_here ? V - ((nch - 1) * EPC - rc.head) : 0;
  tk.xe = -__builtin_inff();
  if (lane < eh) tk.xe = TI::load(row, lane);
  else if (lane - eh < et) tk.xe = TI::load(row, V - et + (lane - eh));
  const int seg_span = 64 * NCH;
  float* rs = (float*)(p.stat + tk.pos);
  if (lane == 0) {
    if ((rc.head + p.blank) / EPC / seg_span == seg) rs[0] = TI::load(row, p.blank);
    int y = -1;
    if (u < U) {
      const int64_t yy = p.labels[(int64_t)b * p.lab_stride + u];
      if (yy >= 0 && yy < V) y = (int)yy;
    }
    if (y >= 0 ? (rc.head + y) / EPC / seg_span == seg : seg == 0)
      rs[1] = y >= 0 ? TI::load(row, y) : -__builtin_inff();
  }
}

template <typename TI, int NCH>
__device__ __forceinline__ void row_task_finish(const Params& p, int lane, RowTask<TI, NCH>& tk) {
  constexpr int EPC = TI::kEpc;
  if (!tk.ok) return;
  const int c0 = tk.c0, nwin = tk.nwin, nch = tk.nch;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int cw = c0 + 64 * j;
    if (j < nwin && (cw == 0 || cw + 63 >= nch - 1)) {
      const int c = cw + lane;
      if (c == 0 || c >= nch - 1) tk.v[j] = neg_inf_chunk<TI>();
    }
  }
  MaxAcc<TI> mx;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    if (j < nwin) {
      mx.add(tk.v[j].x);
      mx.add(tk.v[j].y);
      mx.add(tk.v[j].z);
      mx.add(tk.v[j].w);
    }
  }
  const float xe = tk.xe;
  float mw = wave_max_dpp(fmaxf(mx.value(), xe));
  if constexpr (__is_same(TI, BF16)) {
    if (!(mw >= 0.f)) {
      KeyMaxBF16 km;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        if (j < nwin) {
          km.add(tk.v[j].x);
          km.add(tk.v[j].y);
          km.add(tk.v[j].z);
          km.add(tk.v[j].w);
        }
      }
      mw = wave_max_dpp(fmaxf(km.value(), xe));
    }
  }
  const float c = EPC == 4 ? mw : mw * kLog2e;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    if (j < nwin) {
#pragma unroll
      for (int s = 0; s < EPC; ++s) {
        const float e2 = __builtin_amdgcn_exp2f(expo<TI>(TI::get(tk.v[j], s), c));
        if ((s & 3) == 0) a0 += e2;
        else if ((s & 3) == 1) a1 += e2;
        else if ((s & 3) == 2) a2 += e2;
        else a3 += e2;
      }
    }
  }
  float acc = ((a0 + a1) + (a2 + a3)) + __builtin_amdgcn_exp2f(expo<TI>(xe, c));
  const bool empty = !(mw > -__builtin_inff());
  if (empty) acc = 0.f;
  double S = wave_sum_dpp((double)acc);
  if (!empty && !(__builtin_fabsf(c) < __builtin_inff())) S = __builtin_nan("");
  if (lane == 0) {
    float* part = p.part + (tk.pos * p.nseg + tk.seg) * 2;
    part[0] = empty ? -__builtin_inff() : c;
    part[1] = (float)S;
  }
}

template <typename TI, int NCH>
__global__ __launch_bounds__(256) void k_row_partial2(const Params p) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (blockIdx.x == 0)  // the flags the node-weight kernel of this call sets
    for (int i = threadIdx.x; i < p.B; i += blockDim.x) p.xflag[i] = 0;
  const uint32_t total = (uint32_t)p.B * (uint32_t)p.Tmax * (uint32_t)p.U1max * (uint32_t)p.nseg;
  const uint32_t stride = gridDim.x * kWavesPerBlock;
  for (uint32_t g = xcd_block(blockIdx.x, gridDim.x) * kWavesPerBlock + wv; g < total; g += 2 * stride) {
    RowTask<TI, NCH> t0, t1;
    row_task_load<TI, NCH>(p, g, total, lane, t0);
    row_task_load<TI, NCH>(p, g + stride, total, lane, t1);
    row_task_finish<TI, NCH>(p, lane, t0);
    row_task_finish<TI, NCH>(p, lane, t1);
  }
}

// Gradient value w O softmax(h)_v of one element from its node's record:
//   fp32:   A 2^((x - m) log2e),  A = w O 2^-K, m the row maximum;
//   16-bit: 2^(x log2e - C),      C = c + K - log2|w O| (one fma and one exp2), with the
//           sign of w O (held in A) applied by the caller.
template <typename TI>
__device__ __forceinline__ float grad_val(float x, float A, float m) {
  if constexpr (TI::kEpc == 4) return A * __builtin_amdgcn_exp2f((x - m) * kLog2e);
  else return __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -m));
}

// Gradient of one row segment (natural node order over the padded [B, Tmax, U1max]):
// grad_val for every column, with the blank and label columns and the D duration
// gradients taken from the per-node record (computed in float64 from the lattice).
// Padded nodes and utterances without gradient get zeros.  ALIGNED: the logits row and
// the gradient row have the same address modulo 16 bytes (then both use the same
// chunks); otherwise each lane walks single elements.  The host keeps
// B * Tmax * U1max * nseg below 2^31.
template <typename TI, int NCH, bool ALIGNED>
__global__ __launch_bounds__(256) void k_grad(const Params p) {
  constexpr int EPC = TI::kEpc;
  using ET = typename TI::T;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // one wave per (node, segment), nodes in reverse order (the row-statistics pass ends on
  // the last rows; measured the same as natural order, and a persistent grid of two tasks
  // per wave was slower: 183 vs 180 us at B4 T200 U40 V8193 bf16, 434 vs 371 us in fp32)
  const uint32_t nseg = (uint32_t)p.gnseg;
  const uint32_t per = (uint32_t)p.Tmax * (uint32_t)p.U1max;
  const uint32_t total = (uint32_t)p.B * per * nseg;
  const uint32_t gf = xcd_block(blockIdx.x, gridDim.x) * kWavesPerBlock + wv;
  if (gf >= total) return;
  const uint32_t g = total - 1 - gf;
  const uint32_t node = fdiv(g, p.fd_gnseg);
  const int seg = (int)(g - node * nseg);
  const uint32_t b = fdiv(node, p.fd_tu1);
  const uint32_t rem = node - b * per;
  const int t = (int)fdiv(rem, p.fd_u1);
  const int u = (int)(rem - (uint32_t)t * (uint32_t)p.U1max);
  const int V = p.V;

  bool valid = false;
  float A = 0.f, m = 0.f, Gb = 0.f, Gy = 0.f;
  int ycol = -1;
  const float* rec = nullptr;
  // the three per-utterance words in one round trip (an ok utterance has valid lengths)
  const int ok = p.uok[b];
  const int T = (int)p.Tlen[b], U = (int)p.Ulen[b];
  if (ok) {
    if (t < T && u <= U) {
      valid = true;
      rec = (const float*)(p.lg + node_pos(p, (int)b, t, u) * p.LG);
      A = rec[0];
      m = rec[1];
      Gb = rec[2];
      Gy = rec[3];
      ycol = __float_as_int(rec[4]);
    }
  }
  ET* orow = (ET*)p.gtok + ((int64_t)b * p.gs0 + (int64_t)t * p.gs1 + (int64_t)u * p.gs2);
  const ET* irow = (const ET*)p.tok + ((int64_t)b * p.ts0 + (int64_t)t * p.ts1 + (int64_t)u * p.ts2);

  if (ALIGNED) {
    const RowCover oc = row_cover<TI>(orow, V);
    uint4* obase = (uint4*)oc.base;
    const uint4* ibase = (const uint4*)(((uintptr_t)irow) & ~(uintptr_t)15);
    const int head = oc.head, nch = oc.nch;
    const int cb = (head + p.blank) / EPC, sb = (head + p.blank) % EPC;
    const int cy = ycol >= 0 ? (head + ycol) / EPC : -1, sy = ycol >= 0 ? (head + ycol) % EPC : 0;
    const int c0 = seg * 64 * NCH;
    uint4 v[NCH];
    if (valid) {
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int c = c0 + lane + 64 * j;
        if (c < nch) {
          const u32x4 x = __builtin_nontemporal_load((const u32x4*)(ibase + c));
          v[j] = make_uint4(x.x, x.y, x.z, x.w);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int cw = c0 + 64 * j;  // first chunk of the window
      if (cw >= nch) break;
      const int c = cw + lane;
      if (c >= nch) continue;
      float o[EPC];
      if (valid) {
#pragma unroll
        for (int s = 0; s < EPC; ++s) o[s] = grad_val<TI>(TI::get(v[j], s), A, m);
        if (EPC == 8 && A < 0.f) {  // 16-bit: a negative w O (upstream gradient)
#pragma unroll
          for (int s = 0; s < EPC; ++s) o[s] = -o[s];
        }
        if ((unsigned)(cb - cw) < 64u && c == cb) {
#pragma unroll
          for (int s = 0; s < EPC; ++s)
            if (s == sb) o[s] = Gb;
        }
        if ((unsigned)(cy - cw) < 64u && c == cy) {
#pragma unroll
          for (int s = 0; s < EPC; ++s)
            if (s == sy) o[s] = Gy;
        }
      } else {
#pragma unroll
        for (int s = 0; s < EPC; ++s) o[s] = 0.f;
      }
      const int e0 = c * EPC - head;
      // windows away from the row's first and last chunk store whole chunks
      if ((cw > 0 && cw + 63 < nch - 1) || (e0 >= 0 && e0 + EPC <= V)) {
        const uint4 q = TI::pack(o);
        __builtin_nontemporal_store(u32x4{q.x, q.y, q.z, q.w}, (u32x4*)(obase + c));
      } else {
        ET* oe = (ET*)(obase + c);
#pragma unroll
        for (int s = 0; s < EPC; ++s) {
          const int e = e0 + s;
          if (e >= 0 && e < V) TI::store(oe, s, o[s]);
        }
      }
    }
  } else {
    const int span = 64 * NCH * EPC;
    const int e_end = min(V, (seg + 1) * span);
    for (int e = seg * span + lane; e < e_end; e += 64) {
      float o = 0.f;
      if (valid) {
        o = grad_val<TI>(TI::load(irow, e), A, m);
        if (EPC == 8 && A < 0.f) o = -o;
        if (e == p.blank) o = Gb;
        if (e == ycol) o = Gy;
      }
      TI::store(orow, e, o);
    }
  }
  if (seg == 0 && lane < p.D) {
    const float gd = valid ? rec[5 + lane] : 0.f;
    TI::store(p.gdur, (int64_t)b * p.gds0 + (int64_t)t * p.gds1 + (int64_t)u * p.gds2 + lane, gd);
  }
}

// Segment split of a row of V elements: nseg segments of 64 x nch chunks, nch <= maxw
// (<= 8).  The row-statistics pass takes segments of up to 8 windows of 64 chunks, the
// gradient pass of up to 4.  Measured (ms per step, gradient pass us) for a maximum of
// 2 / 3 / 4 / 6 gradient windows: B4 T200 U40 V8193 bf16 0.338 173 / 0.333 170 /
// 0.333 170 / 0.341 179; the same in fp32 0.618 350 / 0.635 368 / 0.635 367 / 0.635 367;
// the ragged fp16 batch 1.177 660 / 1.006 489 / 1.005 489 / 1.005 488.  The
// row-statistics pass with 4 windows: 146 vs 102 us.
constexpr int kRowWindows = 8;
constexpr int kGradWindows = 4;

inline void pick_segments(int64_t V, int epc, int maxw, int* nch, int* nseg) {
  const int64_t chunks = (V + epc - 1) / epc + 1;
  int64_t s = (chunks + 64 * maxw - 1) / (64 * maxw);
  int64_t n = (chunks + 64 * s - 1) / (64 * s);
  *nseg = (int)s;
  *nch = (int)n;
}

template <typename TI>
hipError_t launch_rows_t(const Params& p, bool aligned, hipStream_t st, int which) {
  const int nch = which == 0 ? p.nch : p.gnch;
  const int64_t nodes = (int64_t)p.B * p.Tmax * p.U1max;  // both passes walk the padded rows
  const int64_t waves = nodes * (which == 0 ? p.nseg : p.gnseg);
  int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  if (which == 0) {  // persistent row statistics
    blocks = (waves + kRowStatTasksPerWave * kWavesPerBlock - 1) / (kRowStatTasksPerWave * kWavesPerBlock);
    if (blocks > kRowStatBlocks) blocks = kRowStatBlocks;
  }
  const dim3 grid((unsigned)blocks);
  if (which == 0) {
#define TDT_RS2(N) \
  case N: hipLaunchKernelGGL((k_row_partial2<TI, N>), grid, dim3(256), 0, st, p); break;
#define TDT_RS(N) \
  case N: hipLaunchKernelGGL((k_row_partial<TI, N>), grid, dim3(256), 0, st, p); break;
    // short segments: the two-task form (see k_row_partial2)
    switch (nch) { TDT_RS2(1) TDT_RS2(2) TDT_RS2(3) TDT_RS2(4) TDT_RS(5) TDT_RS(6) TDT_RS(7) default: TDT_RS(8) }
#undef TDT_RS
#undef TDT_RS2
  } else {
#define TDT_GR(N)                                                                           \
  case N:                                                                                   \
    if (aligned) hipLaunchKernelGGL((k_grad<TI, N, true>), grid, dim3(256), 0, st, p);      \
    else hipLaunchKernelGGL((k_grad<TI, N, false>), grid, dim3(256), 0, st, p);             \
    break;
    switch (nch) { TDT_GR(1) TDT_GR(2) TDT_GR(3) TDT_GR(4) TDT_GR(5) TDT_GR(6) TDT_GR(7) default: TDT_GR(8) }
#undef TDT_GR
  }
  return hipGetLastError();
}

}  // namespace tdt
