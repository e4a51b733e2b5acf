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
// Grid of the persistent row-statistics pass: one (node, segment) task per wave, at most
// 65536 blocks (256K waves; larger batches loop).  Measured row pass, B4 T200 U40 V8193
// bf16 (98,400 tasks) / fp32 (164,000 tasks): one task per wave 83.0 / 157.0 us; two
// 84.5 / 161.7; three 87.5 / 163.9; two with at most 12288 blocks 84.6 / 177.0.
constexpr int kRowStatBlocks = 65536;
constexpr int kRowStatTasksPerWave = 1;
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

// Keep slots [lo, hi) of a chunk and replace the others by -inf.
template <typename TI>
__device__ __forceinline__ uint4 mask_slots(uint4 c, int lo, int hi) {
  uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if constexpr (TI::kEpc == 4) {
      w[q] = (q >= lo && q < hi) ? w[q] : TI::kNegInf;
    } else {
      const bool k0 = 2 * q >= lo && 2 * q < hi, k1 = 2 * q + 1 >= lo && 2 * q + 1 < hi;
      w[q] = (k0 ? (w[q] & 0xffffu) : TI::kNegInf) | (k1 ? (w[q] & 0xffff0000u) : (TI::kNegInf << 16));
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Partial log-sum-exp of one row segment.  Writes, per (node, segment):
//   part[2*seg] = c, part[2*seg + 1] = sum 2^expo(h, c)
// (floats, in a [positions][2*nseg] array).  A segment is NCH windows of 64 16-byte
// chunks, one chunk per lane per window.  The first and the last chunk of the row may hold
// elements of neighbouring rows: their slots outside the row are masked.  A task makes one
// round trip to memory (plus the utterance's lengths, scalar loads).  It is split into its
// index arithmetic (row_task_load), its loads (row_task_issue) and its reductions
// (row_task_finish), so that a wave can issue the loads of two tasks before reducing
// either.
template <typename TI, int NCH>
struct RowTask {
  bool ok;  // a node of its utterance's lattice (wave-uniform)
  bool nt;  // its row is read with nontemporal loads (node < nt_nodes)
  int seg, c0, nch, head;
  int64_t pos;  // node-major index (b, t, u) of the node: its row partials' place
  __amdgpu_buffer_rsrc_t rsrc;
  uint4 v[NCH];
};

// Index arithmetic, lengths, label and buffer resource of a task.
template <typename TI, int NCH>
__device__ __forceinline__ void row_task_load(const Params& p, uint32_t g, uint32_t total, int lane,
                                              RowTask<TI, NCH>& tk) {
  constexpr int EPC = TI::kEpc;
  using ET = typename TI::T;
  tk.ok = false;
  tk.nt = false;
  // a task that is no node of its utterance loads nothing: an empty buffer range
  tk.rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)p.tok, (short)0, 0, 0x00020000);
  tk.c0 = 0;
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
  tk.nt = node < p.nt_nodes;
  tk.seg = seg;
  tk.pos = node;  // node-major index (b, t, u) of the padded box
  const int V = p.V;
  const ET* row = (const ET*)p.tok + ((int64_t)b * p.ts0 + (int64_t)t * p.ts1 + (int64_t)u * p.ts2);
  const RowCover rc = row_cover<TI>(row, V);
  const int nch = rc.nch;
  const int c0 = seg * 64 * NCH;
  tk.nch = nch;
  tk.c0 = c0;
  tk.head = rc.head;
  // range-checked loads (row_task_issue): chunks at or past the end of the row's cover
  // read as zero bits without a memory access (and are masked in row_task_finish)
  tk.rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)rc.base, (short)0, nch * 16, 0x00020000);
}

// The chunk loads of a task; every window is loaded (a task without a node has an empty
// range and reads zeros without a memory access), so the loads of consecutive tasks issue
// back to back.  Nontemporal or ordinary by the task's row (a wave-uniform branch; the
// cache policy is an immediate operand, so the two loops stay apart).
template <typename TI, int NCH>
__device__ __forceinline__ void row_task_issue(int lane, RowTask<TI, NCH>& tk) {
  if (tk.nt) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(tk.rsrc, (tk.c0 + lane + 64 * j) * 16, 0, 2);
      tk.v[j] = make_uint4(x.x, x.y, x.z, x.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(tk.rsrc, (tk.c0 + lane + 64 * j) * 16, 0, 0);
      tk.v[j] = make_uint4(x.x, x.y, x.z, x.w);
    }
  }
}

template <typename TI, int NCH>
__device__ __forceinline__ void row_task_finish(const Params& p, int lane, RowTask<TI, NCH>& tk) {
  constexpr int EPC = TI::kEpc;
  if (!tk.ok) return;
  const int c0 = tk.c0, nch = tk.nch, head = tk.head;
  // slots outside the row: before it in chunk 0, after it in chunk nch-1, and every
  // chunk past the row's cover.  Every window takes part below, also those past the row
  // (all -inf then): a loaded value left unused would make the next loop iteration wait
  // for every load in flight before reusing its register.
  const int tailn = head + p.V - (nch - 1) * EPC;  // slots of chunk nch-1 inside the row
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int cw = c0 + 64 * j;
    if (cw == 0 || cw + 63 >= nch - 1) {
      const int c = cw + lane;
      if (c >= nch) {
        tk.v[j] = neg_inf_chunk<TI>();
      } else {
        const int lo = c == 0 ? head : 0, hi = c == nch - 1 ? tailn : EPC;
        if (lo > 0 || hi < EPC) tk.v[j] = mask_slots<TI>(tk.v[j], lo, hi);
      }
    }
  }
  MaxAcc<TI> mx;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    mx.add(tk.v[j].x);
    mx.add(tk.v[j].y);
    mx.add(tk.v[j].z);
    mx.add(tk.v[j].w);
  }
  float mw = wave_max_dpp(mx.value());
  if constexpr (__is_same(TI, BF16)) {
    if (!(mw >= 0.f)) {  // no non-negative value in the segment: exact maximum from keys
      KeyMaxBF16 km;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        km.add(tk.v[j].x);
        km.add(tk.v[j].y);
        km.add(tk.v[j].z);
        km.add(tk.v[j].w);
      }
      mw = wave_max_dpp(km.value());
    }
  }
  // the shift: the maximum itself (fp32) or maximum * log2e rounded to float (16-bit)
  const float c = EPC == 4 ? mw : mw * kLog2e;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
#pragma unroll
    for (int s = 0; s < EPC; ++s) {
      const float e2 = __builtin_amdgcn_exp2f(expo<TI>(TI::get(tk.v[j], s), c));
      if ((s & 3) == 0) a0 += e2;
      else if ((s & 3) == 1) a1 += e2;
      else if ((s & 3) == 2) a2 += e2;
      else a3 += e2;
    }
  }
  float acc = (a0 + a1) + (a2 + a3);
  const bool empty = !(mw > -__builtin_inff());  // every slot masked: an empty segment
  if (empty) acc = 0.f;
  double S = wave_sum_dpp((double)acc);
  // 16-bit logits beyond about 2.3e38 in magnitude leave no float shift: NaN partial
  if (!empty && !(__builtin_fabsf(c) < __builtin_inff())) S = __builtin_nan("");
  if (lane == 0) {
    float* part = p.part + (tk.pos * p.nseg + tk.seg) * 2;
    part[0] = empty ? -__builtin_inff() : c;
    part[1] = (float)S;
  }
}

// Row statistics, one task at a time (long segments: 5 to 8 windows).  A persistent grid
// of waves walks the (node, segment) space of the padded [B, Tmax, U1max] rows in memory
// order, skipping nodes outside their utterance in a few instructions (ragged batches
// leave most of the padded space empty); the host keeps this space below 2^31.
template <typename TI, int NCH>
__global__ __launch_bounds__(256) void k_row_partial(const Params p) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (blockIdx.x == 0)  // the flags the node-weight kernel of this call sets
    for (int i = threadIdx.x; i < p.B; i += blockDim.x) p.xflag[i] = 0;
  const uint32_t total = (uint32_t)p.B * (uint32_t)p.Tmax * (uint32_t)p.U1max * (uint32_t)p.nseg;
  const uint32_t stride = gridDim.x * kWavesPerBlock;
  for (uint32_t g = xcd_block(blockIdx.x, gridDim.x) * kWavesPerBlock + wv; g < total; g += stride) {
    RowTask<TI, NCH> t0;
    row_task_load<TI, NCH>(p, g, total, lane, t0);
    row_task_issue<TI, NCH>(lane, t0);
    row_task_finish<TI, NCH>(p, lane, t0);
  }
}

// Row statistics for short segments (at most 4 windows): two tasks per loop iteration,
// the loads of both issued before either is reduced.
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
    row_task_issue<TI, NCH>(lane, t0);
    row_task_issue<TI, NCH>(lane, t1);
    row_task_finish<TI, NCH>(p, lane, t0);
    row_task_finish<TI, NCH>(p, lane, t1);
  }
}

// ---- short rows: a quarter wave per row ----
// Rows of at most 16 CPL chunks (CPL <= 16) take 16 lanes each: lane l of the quarter
// holds chunks l, l + 16, ..., l + 16 (CPL - 1) of its row, so a wave holds four rows and a
// 256-thread block sixteen consecutive nodes of the padded [B, Tmax, U1max] space (one
// contiguous stretch of the joint tensor).  Index arithmetic, masks and reductions (over
// the 16 lanes of a row, DPP within a row of the wave) are shared by the four rows, and a
// row of 130 chunks fills 90% of its lanes (against 68% for 64-chunk windows).

// Lengths of the utterances of a block's 16 nodes (first node n0): scalar loads for the
// first and the last node's utterance; when one utterance's box is smaller than 16 nodes
// (a block may span more than two utterances) every lane loads its own.
struct RowLens {
  int64_t T, U;
};
__device__ __forceinline__ RowLens row_lens(const Params& p, uint32_t n0, uint32_t nodes, uint32_t b) {
  const uint32_t per = (uint32_t)p.Tmax * (uint32_t)p.U1max;
  if (per >= 16) {
    const uint32_t bl = fdiv(n0, p.fd_tu1);
    const uint32_t bh = fdiv(min(n0 + 15u, nodes - 1u), p.fd_tu1);
    const int64_t Tl = p.Tlen[bl], Ul = p.Ulen[bl], Th = p.Tlen[bh], Uh = p.Ulen[bh];
    return b == bl ? RowLens{Tl, Ul} : RowLens{Th, Uh};
  }
  return RowLens{p.Tlen[b], p.Ulen[b]};
}

// 16-lane reductions (every lane of a 16-lane row of the wave gets its row's result; the
// sum is taken in the same order on lane 0 of every row)
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
  return fmaxf(x, dpp_f<0x140>(x));  // row_mirror
}
__device__ __forceinline__ double row16_sum(double x) {
  x += dpp_d<0xB1>(x);
  x += dpp_d<0x4E>(x);
  x += dpp_d<0x141>(x);
  return x + dpp_d<0x140>(x);
}

// Row statistics of row (b, t, u) by the 16 lanes of its quarter wave (valid: a row of its
// utterance's lattice; the others load nothing and store nothing).
template <typename TI, int CPL, bool NT>
__device__ __forceinline__ void row_short_task(const Params& p, int b, int t, int u, bool valid, int l16) {
  constexpr int EPC = TI::kEpc;
  using ET = typename TI::T;
  const int V = p.V;
  const ET* row = (const ET*)p.tok + ((int64_t)b * p.ts0 + (int64_t)t * p.ts1 + (int64_t)u * p.ts2);
  const RowCover rc = row_cover<TI>(row, V);
  const int head = rc.head, nch = rc.nch;
  // chunk loads: addresses clamped into the row's cover (chunks past it are masked below);
  // rows outside their utterance load nothing
  uint4 v[CPL];
  if (valid) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = min(l16 + 16 * j, nch - 1);
      const TDT_GLOBAL u32x4* a = (const TDT_GLOBAL u32x4*)(rc.base + c);
      const u32x4 x = NT ? __builtin_nontemporal_load(a) : *a;
      v[j] = make_uint4(x.x, x.y, x.z, x.w);
    }
  }
  // slots outside the row: before it in chunk 0, after it in chunk nch-1, every chunk past
  const int tailn = head + V - (nch - 1) * EPC;  // slots of chunk nch-1 inside the row
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = l16 + 16 * j;
    if (c >= nch) {
      v[j] = neg_inf_chunk<TI>();
    } else if (c == 0 || c == nch - 1) {
      const int lo = c == 0 ? head : 0, hi = c == nch - 1 ? tailn : EPC;
      v[j] = mask_slots<TI>(v[j], lo, hi);
    }
  }
  MaxAcc<TI> mx;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    mx.add(v[j].x);
    mx.add(v[j].y);
    mx.add(v[j].z);
    mx.add(v[j].w);
  }
  float mw = row16_max(mx.value());
  if constexpr (__is_same(TI, BF16)) {
    if (!(mw >= 0.f)) {  // no non-negative value in the row: exact maximum from keys
      KeyMaxBF16 km;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        km.add(v[j].x);
        km.add(v[j].y);
        km.add(v[j].z);
        km.add(v[j].w);
      }
      mw = row16_max(km.value());
    }
  }
  const float c = EPC == 4 ? mw : mw * kLog2e;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
#pragma unroll
    for (int s = 0; s < EPC; ++s) {
      const float e2 = __builtin_amdgcn_exp2f(expo<TI>(TI::get(v[j], s), c));
      if ((s & 3) == 0) a0 += e2;
      else if ((s & 3) == 1) a1 += e2;
      else if ((s & 3) == 2) a2 += e2;
      else a3 += e2;
    }
  }
  float acc = (a0 + a1) + (a2 + a3);
  const bool empty = !(mw > -__builtin_inff());  // every element -inf
  if (empty) acc = 0.f;
  double S = row16_sum((double)acc);
  if (!empty && !(__builtin_fabsf(c) < __builtin_inff())) S = __builtin_nan("");  // see row_task_finish
  if (valid && l16 == 0) {
    // one segment per row, in node-major order (consecutive rows, consecutive records)
    float* part = p.part + (((int64_t)b * p.Tmax + t) * p.U1max + u) * 2;
    part[0] = empty ? -__builtin_inff() : c;
    part[1] = (float)S;
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
  const int64_t T64 = p.Tlen[b], U64 = p.Ulen[b];
  const int T = (int)T64, U = (int)U64;
  // rows outside the utterance's lattice, when the lattice launch has zeroed them
  if (p.zrows && !(utt_dims_ok(p, T64, U64) && t < T && u <= U)) return;
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
    // chunks counted from the gradient row's 128-byte line, so that a window's store
    // instruction writes whole lines except at the row's ends; the logits are read at the
    // same offsets (the rows are equal modulo 16 bytes)
    const uintptr_t oa = (uintptr_t)orow;
    uint4* obase = (uint4*)(oa & ~(uintptr_t)127);
    const int head = (int)((oa & 127) / sizeof(ET));  // elements of the line before the row
    const int nch = (head + V + EPC - 1) / EPC;       // chunks from the line start to the row end
    const int cfirst = head / EPC;                    // the chunk holding the row's first element
    const uint4* ibase = (const uint4*)((const char*)obase + ((const char*)irow - (const char*)orow));
    const int cb = (head + p.blank) / EPC, sb = (head + p.blank) % EPC;
    const int cy = ycol >= 0 ? (head + ycol) / EPC : -1, sy = ycol >= 0 ? (head + ycol) % EPC : 0;
    const int c0 = seg * 64 * NCH;
    uint4 v[NCH];
    if (valid) {
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int c = c0 + lane + 64 * j;
        if (c >= cfirst && c < nch) {
          const u32x4 x = __builtin_nontemporal_load((const TDT_GLOBAL u32x4*)(ibase + c));
          v[j] = make_uint4(x.x, x.y, x.z, x.w);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int cw = c0 + 64 * j;  // first chunk of the window
      if (cw >= nch) break;
      const int c = cw + lane;
      if (c < cfirst || c >= nch) continue;
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
      if ((cw > cfirst && cw + 63 < nch - 1) || (e0 >= 0 && e0 + EPC <= V)) {
        const uint4 q = TI::pack(o);
        __builtin_nontemporal_store(u32x4{q.x, q.y, q.z, q.w}, (TDT_GLOBAL u32x4*)(obase + c));
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

// Row statistics of short rows, a quarter wave per row.  FRAMES (up to 256 labels): one
// work-group per sixteen rows u = 16 c .. 16 c + 15 of a frame (b, t) of the padded box, so
// that a ragged batch pays for its valid rows only (pieces outside the utterance leave at
// once); otherwise sixteen consecutive nodes per work-group (long label sequences: more
// work-groups in flight).  B16 T400 U1max 101 V1025 fp16: 92 us, against 104 us for one
// work-group per frame walking its rows and 155 us for sixteen consecutive nodes; B2 T1000
// U1max 1501 V1025 bf16 (sixteen nodes): 1.28 vs 1.32 ms for one work-group per frame.
template <typename TI, int CPL, bool FRAMES, bool NT>
__global__ __launch_bounds__(256) void k_row_short(const Params p) {
  if (blockIdx.x == 0)  // the flags the node-weight kernel of this call sets
    for (int i = threadIdx.x; i < p.B; i += blockDim.x) p.xflag[i] = 0;
  const int l16 = threadIdx.x & 15;
  if constexpr (FRAMES) {
    const uint32_t nc = ((uint32_t)p.U1max + 15u) >> 4;  // sixteen-row pieces per frame
    const uint32_t f = blockIdx.x / nc;
    const int c = (int)(blockIdx.x - f * nc);
    const int b = (int)(f / (uint32_t)p.Tmax);
    const int t = (int)(f - (uint32_t)b * (uint32_t)p.Tmax);
    const int64_t T64 = p.Tlen[b], U64 = p.Ulen[b];
    if (!utt_dims_ok(p, T64, U64) || t >= (int)T64 || 16 * c > (int)U64) return;
    const int u = 16 * c + (int)(threadIdx.x >> 4);
    row_short_task<TI, CPL, NT>(p, b, t, u, u <= (int)U64, l16);
  } else {
    const uint32_t per = (uint32_t)p.Tmax * (uint32_t)p.U1max;
    const uint32_t nodes = (uint32_t)p.B * per;
    const uint32_t n0 = blockIdx.x * 16u;
    const uint32_t node = n0 + (threadIdx.x >> 4);
    const uint32_t nd = min(node, nodes - 1u);
    const uint32_t b = fdiv(nd, p.fd_tu1);
    const uint32_t rem = nd - b * per;
    const int t = (int)fdiv(rem, p.fd_u1);
    const int u = (int)(rem - (uint32_t)t * (uint32_t)p.U1max);
    const RowLens ln = row_lens(p, n0, nodes, b);
    const bool valid = node < nodes && utt_dims_ok(p, ln.T, ln.U) && t < (int)ln.T && u <= (int)ln.U;
    row_short_task<TI, CPL, NT>(p, (int)b, t, u, valid, l16);
  }
}

// ---- gradient coefficients of a node, inside the short-row gradient pass ----
// Node n = (t, u) of an utterance with a lattice, by the 16 lanes of its quarter wave:
// lane i < D takes duration index i (value d) and the posteriors of the two moves of
// duration d out of n, blank (d >= 1, to (t + d, u)) and label (to (t + d, u + 1)),
//   gamma(e) = alpha(n) W(e) beta(dest e) / P
// (W rebuilt from the node's log-domain ingredients: exp(lb + lambda_d) in float64, the
// plain weight the lattice read up to rounding, or in extended range for an utterance
// whose weights left the plain range; rebuilding takes two exponentials per lane instead
// of two gathers from the weight blocks: B2 T1000 U1500 V1025 bf16 gradient pass 2.49 ->
// 2.30 ms).
// Sums over the quarter give c_blank, c_label and O = c_blank + c_label (every move out
// of n); then
//   grad h_blank = w (O softmax(h)_blank - c_blank),  grad h_y = w (O softmax(h)_y - c_label),
//   grad g_d = w (O softmax(g)_d - c_d)   (lane i, its own duration),
// and every other column w O softmax(h)_v, streamed from grad_val's A and m.  The long-row
// gradient pass, whose waves each take one segment of a row, reads the same numbers from
// the per-node record the coefficient kernel writes.  Every lane of the quarter calls it
// (the sums run across the quarter); a node that is not `valid` gets zeros.
struct NodeGrad {
  float A, m, Gb, Gy;  // grad_val's scale and shift; the blank and label column gradients
  int ycol;            // the label column (-1: none, or the label is the blank)
  float gd;            // lane i < D: the gradient of duration logit i
};

__device__ __forceinline__ NodeGrad node_grad(const Params& p, int b, int t, int u, int T, int U, int li,
                                              bool valid) {
  const bool has = valid && li < p.D;
  int d = 0;  // the lane's duration value (no dynamic index into the kernel arguments)
#pragma unroll
  for (int j = 0; j < kMaxD; ++j) d = li == j ? p.dval[j] : d;
  const int64_t pos = node_pos(p, b, t, u);
  double gb = 0.0, gy = 0.0, lb = 0.0, ly = 0.0, lam = -__builtin_inf();
  if (valid) {
    const double* lgp = p.lg + pos * p.LG;
    lb = lgp[0];
    ly = lgp[1];
    if (has) lam = lgp[2 + li];
  }
  if (has) {
    const bool plain = p.pw != nullptr && p.xflag[b] == 0;
    const Ext a = xrec_get(p.ar, pos);
    const double rP = 1.0 / p.pm[b];
    const int Pe = p.pe[b];
    if (d >= 1) {
      Ext bt = ext_zero();
      if (t + d < T) bt = xrec_get(p.br, node_pos(p, b, t + d, u));
      else if (t + d == T && u == U) bt = ext_one();
      if (bt.m != 0.0) {
        const Ext w = plain ? Ext{exp(lb + lam), 0} : ext_exp(lb + lam);
        gb = ext_to_double(Ext{a.m * w.m * bt.m * rP, a.e + w.e + bt.e - Pe});
      }
    }
    if (u < U && t + d < T) {
      const Ext bt = xrec_get(p.br, node_pos(p, b, t + d, u + 1));
      if (bt.m != 0.0) {
        const Ext w = plain ? Ext{exp(ly + lam), 0} : ext_exp(ly + lam);
        gy = ext_to_double(Ext{a.m * w.m * bt.m * rP, a.e + w.e + bt.e - Pe});
      }
    }
  }
  const double cb = row16_sum(gb), cl = row16_sum(gy);
  NodeGrad g{0.f, 0.f, 0.f, 0.f, -1, 0.f};
  if (valid) {
    const double O = cb + cl;
    const double wgt = p.gscale ? p.wts[b] * (double)p.gscale[p.red == 0 ? b : 0] : p.wts[b];
    // softmax(h)_blank, softmax(h)_label (sigma added back)
    const double sb = exp(lb + p.sigma), sy = exp(ly + p.sigma);
    const float2 rs = p.stat[pos];
    int y = -1;
    if (u < U) y = (int)p.labels[(int64_t)b * p.lab_stride + u];
    double Gb = wgt * (O * sb - cb);
    const double Gy = wgt * (O * sy - cl);
    if (y == p.blank) {  // both corrections land on the blank column
      Gb -= wgt * cl;
      y = -1;
    }
    const double wO = wgt * O;
    if (p.dtype == 0) {  // A = w O 2^-K and the row maximum
      g.A = (float)(wO * exp2(-(double)rs.y));
      g.m = rs.x;
    } else {  // the sign of w O and C = c + K - log2|w O| (base 2)
      g.A = wO < 0.0 ? -1.f : 1.f;
      g.m = (float)((double)rs.x + (double)rs.y - log2(fabs(wO)));
    }
    g.Gb = (float)Gb;
    g.Gy = (float)Gy;
    g.ycol = y;
    if (has) g.gd = (float)(wgt * (O * exp(lam) - (gb + gy)));
  }
  return g;
}

// Gradient of short rows (as k_row_short: a quarter wave per row; FRAMES, up to 256
// labels: one work-group per sixteen rows of a frame, pieces outside the utterance leave
// at once when the lattice launch has zeroed the padding rows, else sixteen consecutive
// nodes per work-group; the work-groups in reverse order), for logits and gradient rows
// with the same address modulo 16 bytes.  Each quarter computes its node's coefficients
// (node_grad), and the first work-group reduces the loss.  B16 T400 U1max 101 V1025 fp16:
// 218 us with frame pieces, 242 us with sixteen consecutive nodes.  The chunks are counted from the gradient row's 128-byte line, so each
// store instruction writes whole lines (16 lanes x 16 bytes, line-aligned) except at the
// row's ends; the logits are read at the same offsets.  Whole chunks inside the row are
// stored as 16-byte nontemporal stores, the row's first and last chunk element by element.
// The blank and label columns are then overwritten by the lane that stored their chunk
// (same thread, so the element store lands after the chunk store).
template <typename TI, int CPL, bool FRAMES>
__global__ __launch_bounds__(256) void k_grad_short(const Params p) {
  constexpr int EPC = TI::kEpc;
  using ET = typename TI::T;
  // the loss of the batch (the lattice has finished every log P), unless the call writes none
  if (p.loss && blockIdx.x == 0 && threadIdx.x == 0) reduce_loss(p);
  const int l16 = threadIdx.x & 15;
  // work-groups in reverse order: the row-statistics pass ended on the last rows
  const uint32_t blk = gridDim.x - 1u - blockIdx.x;
  uint32_t b;
  int t, u;
  bool in;
  RowLens ln;
  if constexpr (FRAMES) {
    const uint32_t nc = ((uint32_t)p.U1max + 15u) >> 4;
    const uint32_t f = blk / nc;
    const int c = (int)(blk - f * nc);
    b = f / (uint32_t)p.Tmax;
    t = (int)(f - b * (uint32_t)p.Tmax);
    u = 16 * c + (int)(threadIdx.x >> 4);
    in = u < p.U1max;
    ln = RowLens{p.Tlen[b], p.Ulen[b]};
    // a piece outside the utterance's lattice: its rows are zeroed by the lattice launch
    if (p.zrows && (!utt_dims_ok(p, ln.T, ln.U) || t >= (int)ln.T || 16 * c > (int)ln.U)) return;
  } else {
    const uint32_t per = (uint32_t)p.Tmax * (uint32_t)p.U1max;
    const uint32_t nodes = (uint32_t)p.B * per;
    const uint32_t n0 = blk * 16u;
    const uint32_t node = n0 + (threadIdx.x >> 4);
    const uint32_t nd = min(node, nodes - 1u);
    b = fdiv(nd, p.fd_tu1);
    const uint32_t rem = nd - b * per;
    t = (int)fdiv(rem, p.fd_u1);
    u = (int)(rem - (uint32_t)t * (uint32_t)p.U1max);
    in = node < nodes;
    ln = row_lens(p, n0, nodes, b);
  }
  const int ok = p.uok[b];  // an ok utterance has valid lengths
  const bool inside = utt_dims_ok(p, ln.T, ln.U) && t < (int)ln.T && u <= (int)ln.U;
  const bool valid = in && ok && inside;
  // rows outside the utterance's lattice are skipped when the lattice launch has zeroed them
  const bool write = in && (inside || p.zrows == 0);
  const int V = p.V;
  // the node's coefficients from the lattice (every lane of the quarter takes part)
  const NodeGrad ng = node_grad(p, (int)b, t, u, (int)ln.T, (int)ln.U, l16, valid);
  const float A = ng.A, m = ng.m;
  ET* orow = (ET*)p.gtok + ((int64_t)b * p.gs0 + (int64_t)t * p.gs1 + (int64_t)u * p.gs2);
  const ET* irow = (const ET*)p.tok + ((int64_t)b * p.ts0 + (int64_t)t * p.ts1 + (int64_t)u * p.ts2);
  const uintptr_t oa = (uintptr_t)orow;
  uint4* obase = (uint4*)(oa & ~(uintptr_t)127);
  const int head = (int)((oa & 127) / sizeof(ET));     // elements of the line before the row
  const int nch = (head + V + EPC - 1) / EPC;          // chunks from the line start to the row end
  const int cfirst = head / EPC;                       // the chunk holding the row's first element
  // logits chunk at the offset of gradient chunk c (rows equal modulo 16 bytes)
  const uint4* ibase = (const uint4*)((const char*)obase + ((const char*)irow - (const char*)orow));
  uint4 v[CPL];
  if (valid) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = min(max(l16 + 16 * j, cfirst), nch - 1);  // inside the row's chunks
      const u32x4 x = __builtin_nontemporal_load((const TDT_GLOBAL u32x4*)(ibase + c));
      v[j] = make_uint4(x.x, x.y, x.z, x.w);
    }
  }
  if (write) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = l16 + 16 * j;
      if (c >= cfirst && c < nch) {
        float o[EPC];
        if (valid) {
#pragma unroll
          for (int s = 0; s < EPC; ++s) o[s] = grad_val<TI>(TI::get(v[j], s), A, m);
          if (EPC == 8 && A < 0.f) {  // 16-bit: a negative w O (upstream gradient)
#pragma unroll
            for (int s = 0; s < EPC; ++s) o[s] = -o[s];
          }
        } else {
#pragma unroll
          for (int s = 0; s < EPC; ++s) o[s] = 0.f;
        }
        const int e0 = c * EPC - head;
        if (e0 >= 0 && e0 + EPC <= V) {
          const uint4 q = TI::pack(o);
          __builtin_nontemporal_store(u32x4{q.x, q.y, q.z, q.w}, (TDT_GLOBAL u32x4*)(obase + c));
        } else {
          ET* oe = (ET*)(obase + c);
#pragma unroll
          for (int s = 0; s < EPC; ++s) {
            const int e = e0 + s;
            if (e >= 0 && e < V) TI::store(oe, s, o[s]);
          }
        }
      }
    }
    if (valid) {
      if (((head + p.blank) / EPC & 15) == l16) TI::store(orow, p.blank, ng.Gb);
      if (ng.ycol >= 0 && ((head + ng.ycol) / EPC & 15) == l16) TI::store(orow, ng.ycol, ng.Gy);
    }
    if (l16 < p.D)
      TI::store(p.gdur, (int64_t)b * p.gds0 + (int64_t)t * p.gds1 + (int64_t)u * p.gds2 + l16, ng.gd);
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

inline void pick_segments(int64_t V, int epc, int maxw, int extra, int* nch, int* nseg) {
  const int64_t chunks = (V + epc - 1) / epc + extra;
  int64_t s = (chunks + 64 * maxw - 1) / (64 * maxw);
  int64_t n = (chunks + 64 * s - 1) / (64 * s);
  *nseg = (int)s;
  *nch = (int)n;
}

// Rows whose cover has at most this many 16-byte chunks take the quarter-wave kernels.
constexpr int kShortRowChunks = 256;

template <typename TI>
hipError_t launch_short_rows(const Params& p, bool aligned, hipStream_t st, int which, int cpl) {
  const int64_t nodes = (int64_t)p.B * p.Tmax * p.U1max;
  // one work-group per sixteen rows of a frame (up to 256 labels) or per sixteen nodes
  const bool frames = p.U1max <= 256;
  const dim3 grid((unsigned)(frames ? (int64_t)p.B * p.Tmax * ((p.U1max + 15) / 16) : (nodes + 15) / 16));
#define TDT_SR(N)                                                                                 \
  case N:                                                                                         \
    if (which == 0 && frames && p.rows_nt) hipLaunchKernelGGL((k_row_short<TI, N, true, true>), grid, dim3(256), 0, st, p); \
    else if (which == 0 && frames) hipLaunchKernelGGL((k_row_short<TI, N, true, false>), grid, dim3(256), 0, st, p); \
    else if (which == 0 && p.rows_nt) hipLaunchKernelGGL((k_row_short<TI, N, false, true>), grid, dim3(256), 0, st, p); \
    else if (which == 0) hipLaunchKernelGGL((k_row_short<TI, N, false, false>), grid, dim3(256), 0, st, p); \
    else if (frames) hipLaunchKernelGGL((k_grad_short<TI, N, true>), grid, dim3(256), 0, st, p); \
    else hipLaunchKernelGGL((k_grad_short<TI, N, false>), grid, dim3(256), 0, st, p); \
    break;
  switch (cpl) {
    TDT_SR(1) TDT_SR(2) TDT_SR(3) TDT_SR(4) TDT_SR(5) TDT_SR(6) TDT_SR(7) TDT_SR(8)
    TDT_SR(9) TDT_SR(10) TDT_SR(11) TDT_SR(12) TDT_SR(13) TDT_SR(14) TDT_SR(15) default: TDT_SR(16)
  }
#undef TDT_SR
  (void)aligned;
  return hipGetLastError();
}

// The gradient pass takes the short-row kernel, which computes the node coefficients
// itself (the coefficient kernel is then left out): rows of at most kShortRowChunks
// chunks counted from their 128-byte line, logits and gradient rows equal modulo 16 bytes.
inline bool short_grad_rows(const Params& p, bool aligned) {
  const int64_t epc = p.dtype == 0 ? 4 : 8;  // elements per 16-byte chunk
  return aligned && ((int64_t)p.V + epc - 1) / epc + 8 <= kShortRowChunks;
}

template <typename TI>
hipError_t launch_rows_t(const Params& p, bool aligned, hipStream_t st, int which) {
  // chunks of a row's cover: from its 16-byte chunk (row statistics) or from its 128-byte
  // line (gradient)
  const int64_t chunks = ((int64_t)p.V + TI::kEpc - 1) / TI::kEpc + (which == 0 ? 1 : 8);
  if (which == 0 ? chunks <= kShortRowChunks : short_grad_rows(p, aligned))
    return launch_short_rows<TI>(p, aligned, st, which, (int)((chunks + 15) / 16));
  const int nch = which == 0 ? p.nch : p.gnch;
  const int64_t nodes = (int64_t)p.B * p.Tmax * p.U1max;  // both passes walk the padded rows
  const int64_t waves = nodes * (which == 0 ? p.nseg : p.gnseg);
  int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  if (which == 0) {  // persistent row statistics (the two-task form: two tasks per wave)
    const int64_t tpw = nch <= 4 ? 2 : kRowStatTasksPerWave;
    blocks = (waves + tpw * kWavesPerBlock - 1) / (tpw * kWavesPerBlock);
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
