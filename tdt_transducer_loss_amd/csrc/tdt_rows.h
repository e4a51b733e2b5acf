// Streaming passes over the token-logit rows of the joint output:
//   row partials — per row segment, the log-sum-exp partial of the V token logits
//                  (the per-node log-softmax of the page "tdt-loss: add TDT loss
//                  kernel", comment "What's in it"), plus the blank and label logits;
//   gradient     — d loss / d token logit for every column of every node, zeros at
//                  padded nodes, written in the logits' dtype (the fused gradient
//                  kernel of the same comment).
//
// A row of V elements is covered by the 16-byte aligned chunks that overlap it (an
// aligned chunk holding a byte of the row never leaves that row's page); head and tail
// slots are masked on reads and written slot by slot.  A row is split into `nseg`
// segments of 64 x NCH chunks, one 64-lane wave per segment, so that a wave keeps at
// most 8 chunks (32 VGPRs) of raw data in flight and many waves fit on each SIMD.
#pragma once

#include "tdt_common.h"

namespace tdt {

constexpr int kWavesPerBlock = 4;   // 256-thread work-groups
constexpr int kRowStatBlocks = 4096;  // grid of the persistent row-statistics pass (16K waves)

template <typename TI>
__device__ __forceinline__ uint4 neg_inf_chunk() {
  const uint32_t w = TI::kEpc == 4 ? TI::kNegInf : (TI::kNegInf | (TI::kNegInf << 16));
  return make_uint4(w, w, w, w);
}

// Running maximum of the raw chunk words, in a form that shares no arithmetic with the
// float decode of the exp pass (so the compiler keeps only the raw words alive).
//   fp32: float max;  fp16: packed half max;  bf16: packed int16 max of order-preserving
//   keys (negative values get their magnitude bits flipped).
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
  __device__ __forceinline__ void add(uint32_t w) {
    const s16x2 x = __builtin_bit_cast(s16x2, w);
    const s16x2 key = x ^ ((x >> (short)15) & (short)0x7fff);
    m = __builtin_elementwise_max(m, key);
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

// Partial log-sum-exp of one row segment.  Writes, per (node, segment):
//   part[2*seg] = m = segment maximum, part[2*seg + 1] = sum 2^((h - m) log2e)
// (floats, in a [positions][2*nseg] array), and the blank / label logits into rstat.
// Exponents are formed as (h - m) * log2e: the difference is small for the elements
// that carry the sum, so the rounding of log2e and of the product stays far below a
// float32 ulp of the result whatever the magnitude of the logits.
template <typename TI, int NCH>
__global__ __launch_bounds__(256) void k_row_partial(const Params p) {
  constexpr int EPC = TI::kEpc;
  using ET = typename TI::T;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (blockIdx.x == 0)  // the node-weight kernel that follows sets these flags
    for (int i = threadIdx.x; i < p.B; i += blockDim.x) p.xflag[i] = 0;
  // persistent: a fixed grid of waves walks the (position, segment) space, skipping
  // positions outside their utterance in a few instructions (ragged batches leave most
  // of the padded space empty)
  const int nseg = p.nseg;
  const int64_t per = (int64_t)p.KD * p.WP;
  const int64_t total = (int64_t)p.B * per * nseg;
  const int64_t stride = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t g = (int64_t)xcd_block(blockIdx.x, gridDim.x) * kWavesPerBlock + wv; g < total; g += stride) {
    const int64_t node = g / nseg;
    const int seg = (int)(g - node * nseg);
    const int b = (int)(node / per);
    const int64_t rem = node - (int64_t)b * per;
    const int k = (int)(rem / p.WP);
    const int i = (int)(rem - (int64_t)k * p.WP);
    const int64_t T64 = p.Tlen[b], U64 = p.Ulen[b];
    if (!utt_dims_ok(p, T64, U64)) continue;
    const int T = (int)T64, U = (int)U64;
    if (k >= T + U) continue;
    const int u = diag_ulo(k, T) + i;
    if (u > min(k, U)) continue;
    const int t = k - u;

    int y = -1;
    if (u < U) {
      const int64_t yy = p.labels[(int64_t)b * p.lab_stride + u];
      if (yy >= 0 && yy < p.V) y = (int)yy;
    }
    const int V = p.V;
    const ET* row = (const ET*)p.tok + ((int64_t)b * p.ts0 + (int64_t)t * p.ts1 + (int64_t)u * p.ts2);
    const RowCover rc = row_cover<TI>(row, V);
    const int c0 = seg * 64 * NCH;

    uint4 v[NCH];
  #pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = c0 + lane + 64 * j;
      v[j] = c < rc.nch ? rc.base[c] : neg_inf_chunk<TI>();
    }
    float* rs = (float*)(p.rstat + rem + (int64_t)b * per);
    const int cb = (rc.head + p.blank) / EPC, sb = (rc.head + p.blank) % EPC;
    const int cy = y >= 0 ? (rc.head + y) / EPC : -1, sy = y >= 0 ? (rc.head + y) % EPC : 0;
    MaxAcc<TI> mx;
  #pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = c0 + lane + 64 * j;
      if (c == 0 || c == rc.nch - 1) {
  #pragma unroll
        for (int s = 0; s < EPC; ++s) {
          const int e = c * EPC + s - rc.head;
          if (e < 0 || e >= V) chunk_set<TI>(v[j], s, TI::kNegInf);
        }
      }
      if (c == cb) rs[2] = TI::get(v[j], sb);
      if (c == cy) rs[3] = TI::get(v[j], sy);
      mx.add(v[j].x);
      mx.add(v[j].y);
      mx.add(v[j].z);
      mx.add(v[j].w);
    }
    // lane-local exp sum relative to the lane's own maximum
    const float ml = mx.value();
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  #pragma unroll
    for (int j = 0; j < NCH; ++j) {
  #pragma unroll
      for (int s = 0; s < EPC; ++s) {
        const float e2 = __builtin_amdgcn_exp2f((TI::get(v[j], s) - ml) * kLog2e);
        if ((s & 3) == 0) a0 += e2;
        else if ((s & 3) == 1) a1 += e2;
        else if ((s & 3) == 2) a2 += e2;
        else a3 += e2;
      }
    }
    float acc = (a0 + a1) + (a2 + a3);
    if (!(ml > -__builtin_inff())) acc = 0.f;  // a lane holding only masked slots
    const float mw = wave_max_f32(ml);
    const float scaled = acc > 0.f ? acc * __builtin_amdgcn_exp2f((ml - mw) * kLog2e) : 0.f;
    const double S = wave_sum_f64((double)scaled);
    if (lane == 0) {
      float* part = p.part + (rem + (int64_t)b * per) * 2 * nseg + 2 * seg;
      part[0] = mw;
      part[1] = (float)S;
      if (seg == 0 && y < 0) rs[3] = -__builtin_inff();
    }
  }
}

// Gradient of one row segment (natural node order over the padded [B, Tmax, U1max]):
//   grad_v = w O softmax(h)_v  computed as  A' * 2^((h_v - m) log2e),  A' = w O 2^-K,
// with the blank and label columns and the D duration gradients taken from the per-node
// record (computed in float64 from the lattice).  Padded nodes and utterances without
// gradient get zeros.  ALIGNED: the logits row and the gradient row have the same
// address modulo 16 bytes (then both use the same chunks); otherwise each lane walks
// single elements.
template <typename TI, int NCH, bool ALIGNED>
__global__ __launch_bounds__(256) void k_grad(const Params p) {
  constexpr int EPC = TI::kEpc;
  using ET = typename TI::T;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t g = (int64_t)xcd_block(blockIdx.x, gridDim.x) * kWavesPerBlock + wv;
  const int nseg = p.nseg;
  const int64_t node = g / nseg;
  const int seg = (int)(g - node * nseg);
  const int64_t per = (int64_t)p.Tmax * p.U1max;
  const int b = (int)(node / per);
  if (b >= p.B) return;
  const int64_t rem = node - (int64_t)b * per;
  const int t = (int)(rem / p.U1max);
  const int u = (int)(rem - (int64_t)t * p.U1max);
  const int V = p.V;

  bool valid = false;
  float A = 0.f, m = 0.f, Gb = 0.f, Gy = 0.f;
  int ycol = -1;
  const float* rec = nullptr;
  if (p.uok[b]) {
    const int T = (int)p.Tlen[b], U = (int)p.Ulen[b];
    if (t < T && u <= U) {
      valid = true;
      const int k = t + u;
      rec = p.rec + node_pos(p, b, k, u - diag_ulo(k, T)) * p.RS;
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
      const int c = c0 + lane + 64 * j;
      if (c >= nch) continue;
      float o[EPC];
#pragma unroll
      for (int s = 0; s < EPC; ++s)
        o[s] = valid ? A * __builtin_amdgcn_exp2f((TI::get(v[j], s) - m) * kLog2e) : 0.f;
      if (valid && c == cb) {
#pragma unroll
        for (int s = 0; s < EPC; ++s)
          if (s == sb) o[s] = Gb;
      }
      if (valid && c == cy) {
#pragma unroll
        for (int s = 0; s < EPC; ++s)
          if (s == sy) o[s] = Gy;
      }
      const int e0 = c * EPC - head;
      if (e0 >= 0 && e0 + EPC <= V) {
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
        o = A * __builtin_amdgcn_exp2f((TI::load(irow, e) - m) * kLog2e);
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

// Segment split of a row of V elements: nseg segments of 64 x nch chunks, nch <= 8.
inline void pick_segments(int64_t V, int epc, int* nch, int* nseg) {
  const int64_t chunks = (V + epc - 1) / epc + 1;
  int64_t s = (chunks + 64 * 8 - 1) / (64 * 8);
  int64_t n = (chunks + 64 * s - 1) / (64 * s);
  *nseg = (int)s;
  *nch = (int)n;
}

template <typename TI>
hipError_t launch_rows_t(const Params& p, bool aligned, hipStream_t st, int which) {
  const int nch = p.nch;
  const int64_t nodes = which == 0 ? (int64_t)p.B * p.KD * p.WP : (int64_t)p.B * p.Tmax * p.U1max;
  const int64_t waves = nodes * p.nseg;
  int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  if (which == 0 && blocks > kRowStatBlocks) blocks = kRowStatBlocks;  // persistent row statistics
  const dim3 grid((unsigned)blocks);
  if (which == 0) {
#define TDT_RS(N) \
  case N: hipLaunchKernelGGL((k_row_partial<TI, N>), grid, dim3(256), 0, st, p); break;
    switch (nch) { TDT_RS(1) TDT_RS(2) TDT_RS(3) TDT_RS(4) TDT_RS(5) TDT_RS(6) TDT_RS(7) default: TDT_RS(8) }
#undef TDT_RS
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
