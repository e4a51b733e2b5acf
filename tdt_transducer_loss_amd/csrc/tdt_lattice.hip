// Lattice side of the TDT loss on gfx950:
//   node weights  — duration log-softmax and the extended-range weight of every move out
//                   of a node (thread per node);
//   lattice       — float64 alpha and beta sweeps over the T x (U+1) lattice, one
//                   work-group per (utterance, direction), anti-diagonal wavefront with
//                   the label index across lanes (the alpha/beta passes of the page
//                   "tdt-loss: add TDT loss kernel", comment "What's in it": float64,
//                   no 1024-label limit);
//   coefficients  — posteriors of the moves out of each node and the per-node record of
//                   the gradient pass, plus the loss reduction.
//
// Probabilities are kept in the linear domain as extended-range float64 (mantissa and a
// separate int exponent), so a lattice step is multiply-adds and exponent arithmetic
// with no exp/log on the serial chain.
#include "tdt_kernels.h"

namespace tdt {

// Reduction weight w_b of utterance b (d reduced loss / d loss_b).
__device__ double reduction_weight(const Params& p, int b, int64_t sumU) {
  switch (p.red) {
    case 3: return 1.0 / (double)p.B;                                        // mean_batch
    case 2: { int64_t U = p.Ulen[b]; return 1.0 / ((double)p.B * (double)(U > 1 ? U : 1)); }  // mean
    case 4: return 1.0 / (double)(sumU > 1 ? sumU : 1);                      // mean_volume
    default: return 1.0;                                                     // none, sum
  }
}

// ------------------------------------------------------------------------------------
// Node weights: for node n = (t,u)
//   l_blank = h_blank - lse, l_label = h_{y_{u+1}} - lse, lambda = log_softmax(g(n)),
//   W_blank(d) = exp(l_blank - sigma + lambda_d)  (d > 0),
//   W_label(d) = exp(l_label - sigma + lambda_d)  (u < U),
// plus softmax(h)_blank, softmax(h)_label and softmax(g) for the gradient.
template <int DM>
__global__ __launch_bounds__(256) void k_node_weights(const Params p) {
  constexpr int NW = 2 * DM + 1;
  const int64_t g = (int64_t)xcd_block(blockIdx.x, gridDim.x) * 256 + threadIdx.x;
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

  const float4 rs = p.rstat[pos];
  const double L = p.lse[pos];
  const double lb = (double)rs.z - L;
  const double ly = (u < U && rs.w > -__builtin_inff()) ? (double)rs.w - L : -__builtin_inf();

  const int64_t dbase = (int64_t)b * p.ds0 + (int64_t)t * p.ds1 + (int64_t)u * p.ds2;
  double gl[DM + 1];
  double gmax = -__builtin_inf();
#pragma unroll
  for (int d = 0; d <= DM; ++d) {
    const int idx = p.didx[d];
    gl[d] = -__builtin_inf();
    if (idx >= 0) {
      gl[d] = (double)load_dur(p, dbase + idx);
      gmax = fmax(gmax, gl[d]);
    }
  }
  double s = 0.0;
#pragma unroll
  for (int d = 0; d <= DM; ++d)
    if (p.didx[d] >= 0) s += exp(gl[d] - gmax);
  const double lse_g = gmax + log(s);

  double* pr = p.pr + pos * p.NPR;
  pr[0] = exp(lb);
  pr[1] = exp(ly);
  const Ext eb = ext_exp(lb - p.sigma);
  const Ext ey = ext_exp(ly - p.sigma);
  double* wm = p.wm;
  int* we = p.we;
#pragma unroll
  for (int d = 0; d <= DM; ++d) {
    const bool has = p.didx[d] >= 0;
    const double lam = gl[d] - lse_g;
    pr[2 + d] = has ? exp(lam) : 0.0;
    const Ext ed = has ? ext_exp(lam) : ext_zero();
    if (d >= 1) {
      const Ext wb = has ? ext_mul(eb, ed) : ext_zero();
      const int64_t o = w_index(p, b, k, d - 1, i);
      wm[o] = wb.m;
      we[o] = wb.e;
    }
    const Ext wl = (has && u < U) ? ext_mul(ey, ed) : ext_zero();
    const int64_t o = w_index(p, b, k, DM + d, i);
    wm[o] = wl.m;
    we[o] = wl.e;
  }
  (void)NW;
}

// ------------------------------------------------------------------------------------
// Lattice sweeps.  Thread j owns labels u = j*R .. j*R + R - 1.  Step k of the alpha
// sweep computes anti-diagonal k (t = k - u); every dependency lies on diagonals
// k-1 .. k-1-DM, kept in a register ring of S >= DM+1 slots (S even, so the double
// buffer of prefetched weights has a fixed slot per unrolled phase).  The value of the
// neighbouring label index owned by the next thread is exchanged once per step (DPP
// wave shift for one wave, LDS + barrier otherwise).  The beta sweep runs the same
// wavefront from the last diagonal back to (0,0).
template <bool SW>
__device__ __forceinline__ Ext exchange(Ext v, bool from_left, int parity, double* xm, int* xe) {
  if (SW) {
    const long long bitsv = __double_as_longlong(v.m);
    int lo = (int)(bitsv & 0xffffffffll), hi = (int)(bitsv >> 32);
    int e = v.e;
    if (from_left) {  // lane i receives lane i-1 (wave_shr:1); lane 0 receives zero
      lo = __builtin_amdgcn_update_dpp(0, lo, 0x138, 0xf, 0xf, false);
      hi = __builtin_amdgcn_update_dpp(0, hi, 0x138, 0xf, 0xf, false);
      e = __builtin_amdgcn_update_dpp(kEZ, e, 0x138, 0xf, 0xf, false);
    } else {          // lane i receives lane i+1 (wave_shl:1); lane 63 receives zero
      lo = __builtin_amdgcn_update_dpp(0, lo, 0x130, 0xf, 0xf, false);
      hi = __builtin_amdgcn_update_dpp(0, hi, 0x130, 0xf, 0xf, false);
      e = __builtin_amdgcn_update_dpp(kEZ, e, 0x130, 0xf, 0xf, false);
    }
    const long long nb = ((long long)(unsigned)hi << 32) | (unsigned)lo;
    return Ext{__longlong_as_double(nb), e};
  } else {
    const int tid = threadIdx.x, nt = blockDim.x;
    xm[parity * 1024 + tid] = v.m;
    xe[parity * 1024 + tid] = v.e;
    __syncthreads();
    const int src = from_left ? tid - 1 : tid + 1;
    if (src < 0 || src >= nt) return ext_zero();
    return Ext{xm[parity * 1024 + src], xe[parity * 1024 + src]};
  }
}

__device__ __forceinline__ Ext load_ext(const Params& p, int64_t o) { return Ext{p.wm[o], p.we[o]}; }

template <int DM, int R, bool SW>
__device__ void alpha_sweep(const Params& p, int b, int T, int U, double* xm, int* xe) {
  constexpr int NW = 2 * DM + 1;
  constexpr int S = ((DM + 2) / 2) * 2;
  const int tid = threadIdx.x;
  const int nsteps = T + U;
  Ext h[R][S];
  Ext nb[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    nb[s] = ext_zero();
#pragma unroll
    for (int r = 0; r < R; ++r) h[r][s] = ext_zero();
  }
  Ext wb[2][R][NW];

  auto load_w = [&](int k, Ext (&w)[R][NW]) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int u = tid * R + r, t = k - u;
      const bool act = t >= 0 && t < T && u <= U;
#pragma unroll
      for (int d = 1; d <= DM; ++d) {
        w[r][d - 1] = ext_zero();
        if (act && t - d >= 0) w[r][d - 1] = load_ext(p, w_index(p, b, k - d, d - 1, u - diag_ulo(k - d, T)));
      }
#pragma unroll
      for (int d = 0; d <= DM; ++d) {
        w[r][DM + d] = ext_zero();
        if (act && u >= 1 && t - d >= 0)
          w[r][DM + d] = load_ext(p, w_index(p, b, k - 1 - d, DM + d, u - 1 - diag_ulo(k - 1 - d, T)));
      }
    }
  };

  load_w(0, wb[0]);
  for (int k0 = 0; k0 < nsteps; k0 += S) {
#pragma unroll
    for (int ph = 0; ph < S; ++ph) {
      const int k = k0 + ph;
      if (k >= nsteps) break;
      if (k + 1 < nsteps) load_w(k + 1, wb[(ph + 1) & 1]);
      Ext nv[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int u = tid * R + r, t = k - u;
        const bool act = t >= 0 && t < T && u <= U;
        Ext terms[NW];
#pragma unroll
        for (int d = 1; d <= DM; ++d) terms[d - 1] = ext_mul(h[r][(ph - d + 4 * S) % S], wb[ph & 1][r][d - 1]);
#pragma unroll
        for (int d = 0; d <= DM; ++d) {
          const Ext src = r > 0 ? h[r > 0 ? r - 1 : 0][(ph - 1 - d + 4 * S) % S] : nb[(ph - 1 - d + 4 * S) % S];
          terms[DM + d] = ext_mul(src, wb[ph & 1][r][DM + d]);
        }
        Ext a = ext_sum(terms);
        if (k == 0 && u == 0) a = ext_one();
        if (!act) a = ext_zero();
        nv[r] = a;
        if (act) {
          const int64_t pos = node_pos(p, b, k, u - diag_ulo(k, T));
          p.am[pos] = a.m;
          p.ae[pos] = a.e;
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) h[r][ph] = nv[r];
      nb[ph] = exchange<SW>(nv[R - 1], true, ph & 1, xm, xe);
    }
  }
  // log P from the alpha side: blanks that land on t = T from u = U
  if (tid * R <= U && U < tid * R + R) {
    __threadfence();
    Ext terms[DM];
#pragma unroll
    for (int d = 1; d <= DM; ++d) {
      terms[d - 1] = ext_zero();
      const int t = T - d;
      if (t >= 0) {
        const int k = t + U;
        const int i = U - diag_ulo(k, T);
        const int64_t pos = node_pos(p, b, k, i);
        terms[d - 1] = ext_mul(Ext{p.am[pos], p.ae[pos]}, load_ext(p, w_index(p, b, k, d - 1, i)));
      }
    }
    p.logpa[b] = ext_log(ext_sum(terms));
  }
}

template <int DM, int R, bool SW>
__device__ void beta_sweep(const Params& p, int b, int T, int U, double* xm, int* xe) {
  constexpr int NW = 2 * DM + 1;
  constexpr int S = ((DM + 2) / 2) * 2;
  const int tid = threadIdx.x;
  const int nsteps = T + U;
  Ext h[R][S];
  Ext nb[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    nb[s] = ext_zero();
#pragma unroll
    for (int r = 0; r < R; ++r) h[r][s] = ext_zero();
  }
  Ext wb[2][R][NW];

  auto load_w = [&](int ks, Ext (&w)[R][NW]) {
    const int k = nsteps - 1 - ks;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int u = tid * R + r, t = k - u;
      const bool act = t >= 0 && t < T && u <= U;
      const int i = u - diag_ulo(k, T);
#pragma unroll
      for (int s = 0; s < NW; ++s) {
        w[r][s] = ext_zero();
        if (act) w[r][s] = load_ext(p, w_index(p, b, k, s, i));
      }
    }
  };

  load_w(0, wb[0]);
  for (int k0 = 0; k0 < nsteps; k0 += S) {
#pragma unroll
    for (int ph = 0; ph < S; ++ph) {
      const int ks = k0 + ph;
      if (ks >= nsteps) break;
      if (ks + 1 < nsteps) load_w(ks + 1, wb[(ph + 1) & 1]);
      const int k = nsteps - 1 - ks;
      Ext nv[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int u = tid * R + r, t = k - u;
        const bool act = t >= 0 && t < T && u <= U;
        Ext terms[NW];
#pragma unroll
        for (int d = 1; d <= DM; ++d) {
          const Ext dst = (t + d == T && u == U) ? ext_one() : h[r][(ph - d + 4 * S) % S];
          terms[d - 1] = ext_mul(dst, wb[ph & 1][r][d - 1]);
        }
#pragma unroll
        for (int d = 0; d <= DM; ++d) {
          const Ext dst = r < R - 1 ? h[r < R - 1 ? r + 1 : 0][(ph - 1 - d + 4 * S) % S] : nb[(ph - 1 - d + 4 * S) % S];
          terms[DM + d] = ext_mul(dst, wb[ph & 1][r][DM + d]);
        }
        Ext a = ext_sum(terms);
        if (!act) a = ext_zero();
        nv[r] = a;
        if (act) {
          const int64_t pos = node_pos(p, b, k, u - diag_ulo(k, T));
          p.bm[pos] = a.m;
          p.be[pos] = a.e;
        }
        if (k == 0 && u == 0) {  // beta(0,0) = P
          const double lp = ext_log(a);
          p.logp[b] = lp;
          p.pm[b] = a.m;
          p.pe[b] = a.e;
          const bool feasible = a.m > 0.0 && lp == lp;
          p.uok[b] = feasible ? 1 : 0;
          if (p.ustatus) p.ustatus[b] = (a.m > 0.0 || lp != lp) ? 0 : 8;
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) h[r][ph] = nv[r];
      nb[ph] = exchange<SW>(nv[0], false, ph & 1, xm, xe);
    }
  }
}

template <int DM, int R, bool SW>
__global__ __launch_bounds__(SW ? 64 : 1024) void k_lattice(const Params p) {
  __shared__ double xm[SW ? 1 : 2 * 1024];
  __shared__ int xe[SW ? 1 : 2 * 1024];
  __shared__ unsigned long long s_sumU;
  const int b = blockIdx.x >> 1, dir = blockIdx.x & 1;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int64_t T64 = p.Tlen[b], U64 = p.Ulen[b];
  int status = 0;
  if (T64 < 0 || T64 > p.Tmax) status |= 1;
  if (U64 < 0 || U64 > p.U1max - 1) status |= 2;
  bool bad = false;
  if (!(status & 2)) {
    for (int64_t u = tid; u < U64; u += nt) {
      const int64_t y = p.labels[(int64_t)b * p.lab_stride + u];
      bad |= (y < 0 || y >= p.V);
    }
  }
  if (tid == 0) s_sumU = 0;
  if (__syncthreads_or(bad)) status |= 4;
  if (dir == 1 && p.red == 4) {
    unsigned long long part = 0;
    for (int bb = tid; bb < p.B; bb += nt) part += (unsigned long long)p.Ulen[bb];
    if (part) atomicAdd(&s_sumU, part);
  }
  __syncthreads();
  if (dir == 1 && tid == 0) p.wts[b] = reduction_weight(p, b, (int64_t)s_sumU);
  const int T = (int)T64, U = (int)U64;
  if (status != 0 || T == 0) {
    if (tid == 0) {
      if (dir == 1) {
        p.logp[b] = status ? __builtin_nan("") : -__builtin_inf();
        p.pm[b] = 0.0;
        p.pe[b] = kEZ;
        p.uok[b] = 0;
        if (p.ustatus) p.ustatus[b] = status ? status : 8;
      } else {
        p.logpa[b] = status ? __builtin_nan("") : -__builtin_inf();
      }
    }
    return;
  }
  if (dir == 0)
    alpha_sweep<DM, R, SW>(p, b, T, U, xm, xe);
  else
    beta_sweep<DM, R, SW>(p, b, T, U, xm, xe);
}

// ------------------------------------------------------------------------------------
// Posteriors and the per-node record of the gradient pass (thread per node):
//   gamma(e) = alpha(n) W(e) beta(dest e) / P,   O(n) = sum over moves out of n,
//   c_blank, c_label = sums over blank / label moves, c_dur(d) = moves of duration d,
//   grad h_blank = w (O softmax(h)_blank - c_blank), grad h_y = w (O softmax(h)_y - c_label),
//   grad g_d = w (O softmax(g)_d - c_dur(d)),  other columns w O softmax(h)_v (streamed).
__device__ void reduce_loss(const Params& p) {
  double s = 0.0;
  for (int b = 0; b < p.B; ++b) {
    const double Lb = -p.logp[b];
    if (p.red == 0)
      p.loss[b] = (float)Lb;
    else
      s += p.wts[b] * Lb;
  }
  if (p.red != 0) p.loss[0] = (float)s;
}

template <int DM>
__global__ __launch_bounds__(256) void k_coef(const Params p) {
  if (blockIdx.x == 0 && threadIdx.x == 0) reduce_loss(p);
  const int64_t g = (int64_t)xcd_block(blockIdx.x, gridDim.x) * 256 + threadIdx.x;
  const int64_t per = (int64_t)p.KD * p.WP;
  const int b = (int)(g / per);
  if (b >= p.B) return;
  if (!p.uok[b]) return;
  const int64_t rem = g - (int64_t)b * per;
  const int k = (int)(rem / p.WP);
  const int i = (int)(rem - (int64_t)k * p.WP);
  const int T = (int)p.Tlen[b], U = (int)p.Ulen[b];
  if (k >= T + U) return;
  const int u = diag_ulo(k, T) + i;
  if (u > min(k, U)) return;
  const int t = k - u;
  const int64_t pos = node_pos(p, b, k, i);

  const Ext a = Ext{p.am[pos], p.ae[pos]};
  const double Pm = p.pm[b];
  const int Pe = p.pe[b];
  double gbl[DM + 1], glb[DM + 1];
  double cb = 0.0, cl = 0.0;
#pragma unroll
  for (int d = 0; d <= DM; ++d) {
    gbl[d] = 0.0;
    glb[d] = 0.0;
    if (d >= 1) {
      Ext bt = ext_zero();
      if (t + d < T) {
        const int k2 = k + d;
        const int64_t o = node_pos(p, b, k2, u - diag_ulo(k2, T));
        bt = Ext{p.bm[o], p.be[o]};
      } else if (t + d == T && u == U) {
        bt = ext_one();
      }
      const Ext w = load_ext(p, w_index(p, b, k, d - 1, i));
      const Ext gm = ext_mul(ext_mul(a, w), bt);
      gbl[d] = ext_to_double(Ext{gm.m / Pm, gm.e - Pe});
      cb += gbl[d];
    }
    if (u < U && t + d < T) {
      const int k2 = k + d + 1;
      const int64_t o = node_pos(p, b, k2, u + 1 - diag_ulo(k2, T));
      const Ext bt = Ext{p.bm[o], p.be[o]};
      const Ext w = load_ext(p, w_index(p, b, k, DM + d, i));
      const Ext gm = ext_mul(ext_mul(a, w), bt);
      glb[d] = ext_to_double(Ext{gm.m / Pm, gm.e - Pe});
      cl += glb[d];
    }
  }
  const double O = cb + cl;
  const double wgt = p.wts[b];
  const double* pr = p.pr + pos * p.NPR;
  const float4 rs = p.rstat[pos];
  int y = -1;
  if (u < U) y = (int)p.labels[(int64_t)b * p.lab_stride + u];
  double Gb = wgt * (O * pr[0] - cb);
  double Gy = wgt * (O * pr[1] - cl);
  if (y == p.blank) {  // both corrections land on the blank column
    Gb -= wgt * cl;
    y = -1;
  }
  float* rec = p.rec + pos * p.RS;
  rec[0] = (float)(wgt * O * exp2(-(double)rs.y));
  rec[1] = rs.x;
  rec[2] = (float)Gb;
  rec[3] = (float)Gy;
  rec[4] = __int_as_float(y);
#pragma unroll
  for (int d = 0; d <= DM; ++d) {
    const int idx = p.didx[d];
    if (idx >= 0) rec[5 + idx] = (float)(wgt * (O * pr[2 + d] - (gbl[d] + glb[d])));
  }
}

__global__ void k_reduce(const Params p) {
  if (threadIdx.x == 0) reduce_loss(p);
}

// ------------------------------------------------------------------------------------
// Launchers
template <int DM>
static hipError_t launch_lattice_dm(const Params& p, hipStream_t st) {
  const int u1 = p.U1max;
  const dim3 grid(2 * p.B);
  if (u1 <= 64) {
    hipLaunchKernelGGL((k_lattice<DM, 1, true>), grid, dim3(64), 0, st, p);
  } else if (u1 <= 128) {
    hipLaunchKernelGGL((k_lattice<DM, 2, true>), grid, dim3(64), 0, st, p);
  } else if (u1 <= 256) {
    hipLaunchKernelGGL((k_lattice<DM, 4, true>), grid, dim3(64), 0, st, p);
  } else {
    int R = u1 <= 1024 ? 1 : u1 <= 2048 ? 2 : u1 <= 4096 ? 4 : 8;
    const int nt = ((u1 + R - 1) / R + 63) / 64 * 64;
    switch (R) {
      case 1: hipLaunchKernelGGL((k_lattice<DM, 1, false>), grid, dim3(nt), 0, st, p); break;
      case 2: hipLaunchKernelGGL((k_lattice<DM, 2, false>), grid, dim3(nt), 0, st, p); break;
      case 4: hipLaunchKernelGGL((k_lattice<DM, 4, false>), grid, dim3(nt), 0, st, p); break;
      default: hipLaunchKernelGGL((k_lattice<DM, 8, false>), grid, dim3(nt), 0, st, p); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_lattice_side(const Params& p, int which, hipStream_t st) {
  const int64_t n = (int64_t)p.B * p.KD * p.WP;
  const dim3 grid((unsigned)((n + 255) / 256));
  switch (which) {
    case 0:  // node weights
      if (p.DM == 4) hipLaunchKernelGGL((k_node_weights<4>), grid, dim3(256), 0, st, p);
      else if (p.DM == 8) hipLaunchKernelGGL((k_node_weights<8>), grid, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((k_node_weights<16>), grid, dim3(256), 0, st, p);
      return hipGetLastError();
    case 1:  // lattice
      if (p.DM == 4) return launch_lattice_dm<4>(p, st);
      if (p.DM == 8) return launch_lattice_dm<8>(p, st);
      return launch_lattice_dm<16>(p, st);
    case 2:  // coefficients + loss
      if (p.DM == 4) hipLaunchKernelGGL((k_coef<4>), grid, dim3(256), 0, st, p);
      else if (p.DM == 8) hipLaunchKernelGGL((k_coef<8>), grid, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((k_coef<16>), grid, dim3(256), 0, st, p);
      return hipGetLastError();
    default:  // loss only
      hipLaunchKernelGGL(k_reduce, dim3(1), dim3(64), 0, st, p);
      return hipGetLastError();
  }
}

}  // namespace tdt
