// Streaming passes over the token-logit rows of the joint output (one 64-lane wave per
// lattice node):
//   row statistics — log-softmax normaliser of the V token logits, plus the blank and
//                    label logits (the per-node log-softmax of the page "tdt-loss: add
//                    TDT loss kernel", comment "What's in it");
//   gradient       — d loss / d token logit for every column of every node, zeros at
//                    padded nodes, written in the logits' dtype (the fused gradient
//                    kernel of the same comment).
//
// Rows are read in place, whatever their alignment: a wave covers the row with the
// 16-byte aligned chunks that overlap it (an aligned chunk holding a byte of the row
// never leaves that row's page), masks the head and tail slots, and writes partial
// chunks slot by slot.
#pragma once

#include "tdt_common.h"

namespace tdt {

constexpr int kRowsPerBlock = 4;  // waves (rows) per 256-thread work-group

template <typename TI>
__device__ __forceinline__ uint4 neg_inf_chunk() {
  const uint32_t w = TI::kEpc == 4 ? TI::kNegInf : (TI::kNegInf | (TI::kNegInf << 16));
  return make_uint4(w, w, w, w);
}

// Statistics of one token row: mL = f32(max * log2e), K = log2 sum_v 2^(h_v log2e - mL),
// lse = (mL + K) ln 2, and the blank / label logits.
template <typename TI, int NCH>
__global__ __launch_bounds__(256) void k_row_stats(const Params p) {
  constexpr int EPC = TI::kEpc;
  using ET = typename TI::T;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t g = (int64_t)xcd_block(blockIdx.x, gridDim.x) * kRowsPerBlock + wv;
  const int64_t per = (int64_t)p.KD * p.WP;
  const int b = (int)(g / per);
  if (b >= p.B) return;
  const int64_t rem = g - (int64_t)b * per;
  const int k = (int)(rem / p.WP);
  const int i = (int)(rem - (int64_t)k * p.WP);
  const int64_t T64 = p.Tlen[b], U64 = p.Ulen[b];
  if (!utt_dims_ok(p, T64, U64)) return;
  const int T = (int)T64, U = (int)U64;
  if (k >= T + U) return;
  const int u = diag_ulo(k, T) + i;
  if (u > min(k, U)) return;
  const int t = k - u;
  const int64_t pos = node_pos(p, b, k, i);

  int y = -1;
  if (u < U) {
    const int64_t yy = p.labels[(int64_t)b * p.lab_stride + u];
    if (yy >= 0 && yy < p.V) y = (int)yy;
  }
  const int V = p.V;
  const char* row = (const char*)p.tok + (int64_t)sizeof(ET) * ((int64_t)b * p.ts0 + (int64_t)t * p.ts1 + (int64_t)u * p.ts2);
  const uintptr_t a = (uintptr_t)row;
  const uint4* base = (const uint4*)(a & ~(uintptr_t)15);
  const int head = (int)((a & 15) / sizeof(ET));
  const int nch = (head + V + EPC - 1) / EPC;
  const int cb = (head + p.blank) / EPC, sb = (head + p.blank) % EPC;
  const int cy = y >= 0 ? (head + y) / EPC : -1, sy = y >= 0 ? (head + y) % EPC : 0;

  float m = -__builtin_inff();
  float mL = -__builtin_inff();
  float acc = 0.f;
  float hb = 0.f, hy = 0.f;
  bool own_b = false, own_y = false;
  for (int c0 = 0; c0 < nch; c0 += 64 * NCH) {
    uint4 v[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = c0 + lane + 64 * j;
      v[j] = c < nch ? base[c] : neg_inf_chunk<TI>();
    }
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = c0 + lane + 64 * j;
      if (c == 0 || c == nch - 1) {
#pragma unroll
        for (int s = 0; s < EPC; ++s) {
          const int e = c * EPC + s - head;
          if (e < 0 || e >= V) chunk_set<TI>(v[j], s, TI::kNegInf);
        }
      }
      if (c == cb) {
        hb = TI::get(v[j], sb);
        own_b = true;
      }
      if (c == cy) {
        hy = TI::get(v[j], sy);
        own_y = true;
      }
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
#pragma unroll
      for (int s = 0; s < EPC; ++s) mx = fmaxf(mx, TI::get(v[j], s));
    }
    mx = wave_max_f32(mx);
    if (mx > m) {  // wave-uniform
      const float mLn = mx * kLog2e;
      acc = acc * __builtin_amdgcn_exp2f(mL - mLn);
      m = mx;
      mL = mLn;
    }
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
#pragma unroll
      for (int s = 0; s < EPC; ++s) {
        const float e2 = __builtin_amdgcn_exp2f(fmaf(TI::get(v[j], s), kLog2e, -mL));
        if ((s & 3) == 0) a0 += e2;
        else if ((s & 3) == 1) a1 += e2;
        else if ((s & 3) == 2) a2 += e2;
        else a3 += e2;
      }
    }
    acc += (a0 + a1) + (a2 + a3);
  }
  const double S = wave_sum_f64((double)acc);
  float* rs = (float*)(p.rstat + pos);
  if (lane == 0) {
    const double K = log2(S);
    rs[0] = mL;
    rs[1] = (float)K;
    p.lse[pos] = ((double)mL + K) * kLn2;
    if (y < 0) rs[3] = -__builtin_inff();
  }
  if (own_b) rs[2] = hb;
  if (own_y) rs[3] = hy;
}

// Gradient of one token row (natural node order over the padded [B, Tmax, U1max]):
//   grad_v = w O softmax(h)_v  computed as  A' * 2^(h_v log2e - mL),  A' = w O 2^-K,
// with the blank and label columns and the D duration gradients taken from the per-node
// record (computed in float64 from the lattice).  Padded nodes and utterances without
// gradient get zeros.  ALIGNED: the logits row and the gradient row have the same
// address modulo 16 bytes (then both use the same chunks).
template <typename TI, int NCH, bool ALIGNED>
__global__ __launch_bounds__(256) void k_grad(const Params p) {
  constexpr int EPC = TI::kEpc;
  using ET = typename TI::T;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t g = (int64_t)xcd_block(blockIdx.x, gridDim.x) * kRowsPerBlock + wv;
  const int64_t per = (int64_t)p.Tmax * p.U1max;
  const int b = (int)(g / per);
  if (b >= p.B) return;
  const int64_t rem = g - (int64_t)b * per;
  const int t = (int)(rem / p.U1max);
  const int u = (int)(rem - (int64_t)t * p.U1max);
  const int V = p.V;

  bool valid = false;
  float A = 0.f, mL = 0.f, Gb = 0.f, Gy = 0.f;
  int ycol = -1;
  const float* rec = nullptr;
  if (p.uok[b]) {
    const int T = (int)p.Tlen[b], U = (int)p.Ulen[b];
    if (t < T && u <= U) {
      valid = true;
      const int k = t + u;
      rec = p.rec + node_pos(p, b, k, u - diag_ulo(k, T)) * p.RS;
      A = rec[0];
      mL = rec[1];
      Gb = rec[2];
      Gy = rec[3];
      ycol = __float_as_int(rec[4]);
    }
  }
  char* orow = (char*)p.gtok + (int64_t)sizeof(ET) * ((int64_t)b * p.gs0 + (int64_t)t * p.gs1 + (int64_t)u * p.gs2);
  const char* irow = (const char*)p.tok + (int64_t)sizeof(ET) * ((int64_t)b * p.ts0 + (int64_t)t * p.ts1 + (int64_t)u * p.ts2);

  if (ALIGNED) {
    const uintptr_t a = (uintptr_t)orow;
    uint4* obase = (uint4*)(a & ~(uintptr_t)15);
    const uint4* ibase = (const uint4*)(((uintptr_t)irow) & ~(uintptr_t)15);
    const int head = (int)((a & 15) / sizeof(ET));
    const int nch = (head + V + EPC - 1) / EPC;
    const int cb = (head + p.blank) / EPC, sb = (head + p.blank) % EPC;
    const int cy = ycol >= 0 ? (head + ycol) / EPC : -1, sy = ycol >= 0 ? (head + ycol) % EPC : 0;
    for (int c0 = 0; c0 < nch; c0 += 64 * NCH) {
      uint4 v[NCH];
      if (valid) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          const int c = c0 + lane + 64 * j;
          if (c < nch) v[j] = ibase[c];
        }
      }
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int c = c0 + lane + 64 * j;
        if (c >= nch) continue;
        float o[EPC];
#pragma unroll
        for (int s = 0; s < EPC; ++s)
          o[s] = valid ? A * __builtin_amdgcn_exp2f(fmaf(TI::get(v[j], s), kLog2e, -mL)) : 0.f;
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
          obase[c] = TI::pack(o);
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
  } else {
    for (int e = lane; e < V; e += 64) {
      float o = 0.f;
      if (valid) {
        o = A * __builtin_amdgcn_exp2f(fmaf(TI::load(irow, e), kLog2e, -mL));
        if (e == p.blank) o = Gb;
        if (e == ycol) o = Gy;
      }
      TI::store(orow, e, o);
    }
  }
  if (lane < p.D) {
    const float gd = valid ? rec[5 + lane] : 0.f;
    TI::store(p.gdur, (int64_t)b * p.gds0 + (int64_t)t * p.gds1 + (int64_t)u * p.gds2 + lane, gd);
  }
}

// Chunks per lane of the row kernels: the smallest variant that covers a row of V
// elements (with its misaligned head) in one pass; wider rows loop over passes.
constexpr int kNchVariants[] = {1, 2, 4, 9, 17, 33};

inline int pick_nch(int64_t V, int epc) {
  const int64_t chunks = (V + epc - 1) / epc + 1;
  for (int n : kNchVariants)
    if (chunks <= 64 * (int64_t)n) return n;
  return 33;
}

template <typename TI>
hipError_t launch_rows_t(const Params& p, bool aligned, hipStream_t st, int which) {
  const int nch = pick_nch(p.V, TI::kEpc);
  if (which == 0) {
    const int64_t waves = (int64_t)p.B * p.KD * p.WP;
    const dim3 grid((unsigned)((waves + kRowsPerBlock - 1) / kRowsPerBlock));
#define TDT_RS(N) \
  case N: hipLaunchKernelGGL((k_row_stats<TI, N>), grid, dim3(256), 0, st, p); break;
    switch (nch) { TDT_RS(1) TDT_RS(2) TDT_RS(4) TDT_RS(9) TDT_RS(17) default: TDT_RS(33) }
#undef TDT_RS
  } else {
    const int64_t waves = (int64_t)p.B * p.Tmax * p.U1max;
    const dim3 grid((unsigned)((waves + kRowsPerBlock - 1) / kRowsPerBlock));
#define TDT_GR(N)                                                              \
  case N:                                                                      \
    if (aligned) hipLaunchKernelGGL((k_grad<TI, N, true>), grid, dim3(256), 0, st, p); \
    else hipLaunchKernelGGL((k_grad<TI, N, false>), grid, dim3(256), 0, st, p);        \
    break;
    switch (nch) { TDT_GR(1) TDT_GR(2) TDT_GR(4) TDT_GR(9) TDT_GR(17) default: TDT_GR(33) }
#undef TDT_GR
  }
  return hipGetLastError();
}

}  // namespace tdt
