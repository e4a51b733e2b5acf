// Lattice side of the TDT loss on gfx950:
//   node weights  — duration log-softmax and the extended-range weight of every move out
//                   of a node (thread per node), stored per node as an outgoing record
//                   and scattered into the incoming record of each destination;
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

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
typedef unsigned int u32x3v __attribute__((ext_vector_type(3)));
// Pointer into LDS (address space 3): stores and loads through it are ds_* operations
// and never wait on outstanding global loads.
typedef __attribute__((address_space(3))) int lds_int;

// Reduction weight w_b of utterance b (d reduced loss / d loss_b).
__device__ double reduction_weight(const Params& p, int b, int64_t sumU) {
  switch (p.red) {
    case 3: return 1.0 / (double)p.Btot;  // mean_batch
    case 2: {                             // mean
      const int64_t U = p.Ulen[b];
      return 1.0 / ((double)p.Btot * (double)(U > 1 ? U : 1));
    }
    case 4: return 1.0 / (double)(sumU > 1 ? sumU : 1);  // mean_volume
    default: return 1.0;                                 // none, sum
  }
}

// ---- records ----
// Weight record of a node (RW bytes, 16-byte aligned): NW float64 mantissas, then NW
// int32 exponents carrying +kWBias (all-zero bits = the zero weight).  Slot d-1
// (d = 1..DM) is the blank move of duration d, slot DM+d (d = 0..DM) the label move of
// duration d.  Alpha / beta records are 16 bytes: float64 mantissa, int32 exponent.
__device__ __forceinline__ char* wrec(char* base, const Params& p, int64_t pos) { return base + pos * p.RW; }

__device__ __forceinline__ void wrec_put(char* rec, int NW, int s, Ext w) {
  ((double*)rec)[s] = w.m;
  ((int*)(rec + 8 * NW))[s] = w.m == 0.0 ? 0 : w.e + kWBias;
}

// A move weight: values in [2^-1000, 2^1000] are stored as plain float64 numbers with a
// zero exponent (exactly), others in extended form.  Returns true when the weight is
// non-zero and outside [2^-300, 2^300], the range the plain-float64 sweep accepts.
__device__ __forceinline__ bool wrec_put_weight(char* rec, int NW, int s, Ext w) {
  if (w.m == 0.0) {
    wrec_put(rec, NW, s, ext_zero());
    return false;
  }
  const Ext n = ext_norm(w.m, w.e);  // value in [2^(e-1), 2^e)
  if (n.e >= -999 && n.e <= 1000) {
    ((double*)rec)[s] = ldexp(n.m, n.e);
    ((int*)(rec + 8 * NW))[s] = kWBias;
  } else {
    wrec_put(rec, NW, s, n);
  }
  return n.e < -299 || n.e > 300;
}

// Slot-pair-major copy of the plain float64 weights for the plain sweeps (empty when one
// utterance's copy would exceed 2 GB): [b][k][slot / 2][column][slot % 2], rows of UW
// columns, label u in column (u % PR) * (UW / PR) + u / PR, so that one 16-byte load per
// lane fetches two slots of one of its R = PR labels and the lanes of a wave read
// consecutive bytes.
__host__ __device__ constexpr int slot_pairs(int NW) { return (NW + 1) / 2; }

__device__ __forceinline__ void pw_put(double* pw, const Params& p, int b, int k, int s, int u, Ext w) {
  if (pw) {
    const int col = (u % p.PR) * (p.UW / p.PR) + u / p.PR;  // label u of lane u / PR
    pw[((((int64_t)b * p.KD + k) * slot_pairs(p.NW) + (s >> 1)) * p.UW + col) * 2 + (s & 1)] =
        w.m == 0.0 ? 0.0 : ldexp(w.m, w.e);
  }
}

__device__ __forceinline__ Ext wrec_get(const char* rec, int NW, int s) {
  return Ext{((const double*)rec)[s], ((const int*)(rec + 8 * NW))[s] - kWBias};
}

__device__ __forceinline__ Ext xrec_get(const char* base, int64_t pos) {
  const char* r = base + pos * 16;
  return Ext{*(const double*)r, *(const int*)(r + 8)};
}

// ------------------------------------------------------------------------------------
// Node weights: for node n = (t,u)
//   l_blank = h_blank - lse, l_label = h_{y_{u+1}} - lse, lambda = log_softmax(g(n)),
//   W_blank(d) = exp(l_blank - sigma + lambda_d)  (d > 0; t+d < T, or t+d = T at u = U),
//   W_label(d) = exp(l_label - sigma + lambda_d)  (u < U, t+d < T),
// plus softmax(h)_blank, softmax(h)_label and softmax(g) for the gradient.  A group of
// NG = 8, 16 or 32 lanes (at least DM + 1) works on one lattice position: lane d of the
// group handles duration value d, lanes 0..3 the per-node exponentials, so the float64
// work of a node is spread over its group.  Every record of a node in the lattice is
// written: moves that leave the lattice, absent durations and moves with no source hold
// the zero weight, so the sweeps read the records of active nodes without predicates.
// Slot s of the incoming record of n is written by the source of that move, or zeroed by
// n itself when the source does not exist (exactly one writer per slot).
template <int DM>
__global__ __launch_bounds__(256) void k_node_weights(const Params p) {
  constexpr int NW = 2 * DM + 1;
  constexpr int NG = DM < 8 ? 8 : (DM < 16 ? 16 : 32);
  const int64_t gt = (int64_t)xcd_block(blockIdx.x, gridDim.x) * 256 + threadIdx.x;
  const int j = threadIdx.x & (NG - 1);  // lane in the group: duration value j
  const int64_t g = gt / NG;              // lattice position of the group
  const int64_t per = (int64_t)p.KD * p.WP;
  const int b = (int)(g / per);
  if (b >= p.B) return;  // whole groups leave together
  const int64_t rem = g - (int64_t)b * per;
  const int k = (int)(rem / p.WP);
  const int i = (int)(rem - (int64_t)k * p.WP);
  const int64_t pos = (int64_t)b * per + rem;
  char* orec = wrec(p.wout, p, pos);
  char* irec = wrec(p.win, p, pos);
  const int64_t T64 = p.Tlen[b], U64 = p.Ulen[b];
  const int T = (int)T64, U = (int)U64;
  const bool dims = utt_dims_ok(p, T64, U64);
  const int u = dims ? diag_ulo(k, T) + i : 0;
  const bool valid = dims && k < T + U && u <= min(k, U);
  const int d = j;
  // positions outside the utterance write nothing: every slot of a node in the lattice
  // is written by the source of its move or zeroed by the node itself, and the sweeps
  // discard whatever lanes outside the lattice compute
  if (!valid) return;
  const int t = k - u;

  // the duration logit of this lane, loaded first
  const int idx = d <= DM ? p.didx[d] : -1;
  const bool has = idx >= 0;
  const int64_t dbase = (int64_t)b * p.ds0 + (int64_t)t * p.ds1 + (int64_t)u * p.ds2;
  const double gl = has ? (double)load_dur(p, dbase + idx) : -__builtin_inf();

  // log-sum-exp of the token logits from the row-segment partials (lane s: segment s);
  // 16-bit logits keep their shifts in base-2 units (see k_row_partial).  A NaN partial
  // (logits beyond the float range of the shift) propagates.
  const bool base2 = p.dtype != 0;
  const float F = base2 ? 1.f : kLog2e;
  const float* part = p.part + pos * 2 * p.nseg;
  float ms = -__builtin_inff();
  float ps = 0.f;
  for (int s2 = j; s2 < p.nseg; s2 += NG) {
    const float m2 = part[2 * s2], p2 = part[2 * s2 + 1];
    if (!(p2 <= 0.f)) {
      const float mn = fmaxf(ms, m2);
      ps = (ps != 0.f ? ps * __builtin_amdgcn_exp2f((ms - mn) * F) : 0.f) + p2 * __builtin_amdgcn_exp2f((m2 - mn) * F);
      ms = mn;
    }
  }
  float mx = ms;
#pragma unroll
  for (int o = NG / 2; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, NG));
  double S = ps != 0.f ? (double)ps * exp2(((double)ms - (double)mx) * (base2 ? 1.0 : kLog2eD)) : 0.0;
#pragma unroll
  for (int o = NG / 2; o >= 1; o >>= 1) S += __shfl_xor(S, o, NG);
  const double K = log2(S);
  const double L = row_lse(base2, (double)mx, K);  // natural-log normaliser
  const float4 rs = p.rstat[pos];
  const double lb = (double)rs.z - L;
  const double ly = (u < U && rs.w > -__builtin_inff()) ? (double)rs.w - L : -__builtin_inf();

  // lanes 0..3: exp(l_blank - sigma), exp(l_label - sigma) in extended range, and
  // softmax(h)_blank, softmax(h)_label
  const double xl = (j & 1) ? ly : lb;
  Ext ex = ext_zero();
  if (j < 2) ex = ext_exp(xl - p.sigma);
  double* pr = p.pr + pos * p.NPR;
  if (j >= 2 && j < 4) pr[j - 2] = exp(xl);
  if (j == 0) ((float2*)(p.rstat + pos))[0] = make_float2(mx, (float)K);
  const int base = threadIdx.x & ~(NG - 1);
  const Ext eb = Ext{__shfl(ex.m, base, 64), __shfl(ex.e, base, 64)};
  const Ext ey = Ext{__shfl(ex.m, base + 1, 64), __shfl(ex.e, base + 1, 64)};

  // duration softmax: lambda_d = gl - gmax - log(sg)
  double gmax = gl;
#pragma unroll
  for (int o = NG / 2; o >= 1; o >>= 1) gmax = fmax(gmax, __shfl_xor(gmax, o, NG));
  const double eg = has ? exp(gl - gmax) : 0.0;
  double sg = eg;
#pragma unroll
  for (int o = NG / 2; o >= 1; o >>= 1) sg += __shfl_xor(sg, o, NG);
  const double pd = eg / sg;
  // exp(lambda_d) in extended range: the quotient unless it left the normal range
  const Ext ed = !has ? ext_zero() : (gl - gmax > -700.0 ? ext_norm(pd, 0) : ext_exp(gl - gmax - log(sg)));

  bool wide = false;
  if (d <= DM) {
    pr[2 + d] = has ? pd : 0.0;
    const int64_t ub = (int64_t)b * per;
    if (d >= 1) {
      const bool inside = t + d < T;
      const bool ok = has && (inside || (t + d == T && u == U));
      const Ext wb = ok ? ext_mul(eb, ed) : ext_zero();
      wide |= wrec_put_weight(orec, NW, d - 1, wb);
      pw_put(p.pwout, p, b, k, d - 1, u, wb);
      if (inside) {  // incoming slot of (t+d, u)
        const int k2 = k + d;
        wrec_put_weight(wrec(p.win, p, ub + (int64_t)k2 * p.WP + (u - diag_ulo(k2, T))), NW, d - 1, wb);
        pw_put(p.pwin, p, b, k2, d - 1, u, wb);
      }
      if (t - d < 0) {  // no source for this slot
        wrec_put(irec, NW, d - 1, ext_zero());
        pw_put(p.pwin, p, b, k, d - 1, u, ext_zero());
      }
    }
    const bool inside = u < U && t + d < T;
    const Ext wl = (has && inside) ? ext_mul(ey, ed) : ext_zero();
    wide |= wrec_put_weight(orec, NW, DM + d, wl);
    pw_put(p.pwout, p, b, k, DM + d, u, wl);
    if (inside) {  // incoming slot of (t+d, u+1)
      const int k2 = k + d + 1;
      wrec_put_weight(wrec(p.win, p, ub + (int64_t)k2 * p.WP + (u + 1 - diag_ulo(k2, T))), NW, DM + d, wl);
      pw_put(p.pwin, p, b, k2, DM + d, u + 1, wl);
    }
    if (u == 0 || t - d < 0) {
      wrec_put(irec, NW, DM + d, ext_zero());
      pw_put(p.pwin, p, b, k, DM + d, u, ext_zero());
    }
  }
  if (wide) atomicOr(p.xflag + b, 1);
}

// ------------------------------------------------------------------------------------
// Lattice sweeps.  Thread j owns labels u = j*R .. j*R + R - 1.  Step k of the alpha
// sweep computes anti-diagonal k (t = k - u); every dependency lies on diagonals
// k-1 .. k-1-DM, kept in a register ring of S >= DM+1 slots.  S is a multiple of 6 so
// that, after unrolling S steps, the exchange parity (2) and the triple buffer of
// weight records prefetched two steps ahead (3) sit in fixed registers.  The value of
// the neighbouring label index owned by the next thread is exchanged once per step (DPP
// wave shift for one wave, LDS + barrier otherwise).  The beta sweep runs the same
// wavefront from the last diagonal back to (0,0).
template <int DM>
__host__ __device__ constexpr int ring_size() { return ((DM + 1 + 5) / 6) * 6; }

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

// Pairwise (tree) reductions for the sum of extended values: shorter dependency chains
// than a running sum, which is what bounds one lattice step.
template <int N>
__device__ __forceinline__ int tree_max_e(const Ext* t) {
  if constexpr (N == 1) return t[0].e;
  else return max(tree_max_e<N / 2>(t), tree_max_e<N - N / 2>(t + N / 2));
}
template <int N>
__device__ __forceinline__ double tree_sum_m(const Ext* t, int E) {
  if constexpr (N == 1) return ldexp(t[0].m, t[0].e - E);
  else return tree_sum_m<N / 2>(t, E) + tree_sum_m<N - N / 2>(t + N / 2, E);
}
// Sum of terms whose exponents all carry +kWBias; returns the un-biased sum.
template <int N>
__device__ __forceinline__ Ext ext_sum_biased(const Ext (&t)[N]) {
  const int E = tree_max_e<N>(t);
  const double sm = tree_sum_m<N>(t, E);
  return ext_norm(sm, E - kWBias);
}

// A weight record loaded as RW/16 16-byte words; decoded slot by slot.
template <int DM>
struct WRec {
  static constexpr int NW = 2 * DM + 1;
  static constexpr int NQ = rec_bytes(DM) / 16;
  u32x4v q[NQ];
  __device__ __forceinline__ uint32_t dw(int j) const { return q[j >> 2][j & 3]; }
  __device__ __forceinline__ Ext get(int s) const {  // biased exponent kept
    const uint64_t bits = ((uint64_t)dw(2 * s + 1) << 32) | dw(2 * s);
    return Ext{__builtin_bit_cast(double, bits), (int)dw(2 * NW + s)};
  }
};

// P = beta(0,0) of utterance b: log P, P as mantissa / exponent, the gradient flag and
// the infeasible status bit.
__device__ void beta_final(const Params& p, int b, Ext P) {
  const double lp = ext_log(P);
  p.logp[b] = lp;
  p.pm[b] = P.m;
  p.pe[b] = P.e;
  const bool feasible = P.m > 0.0 && lp == lp;
  p.uok[b] = feasible ? 1 : 0;
  if (p.ustatus) p.ustatus[b] = (P.m > 0.0 || lp != lp) ? 0 : 8;
}

// log P from the alpha side (the thread that owns u = U, after its last alpha store):
// the blanks that land on t = T from u = U.
template <int DM>
__device__ double alpha_terminal(const Params& p, int b, int T, int U) {
  constexpr int NW = 2 * DM + 1;
  __threadfence();
  Ext terms[DM];
#pragma unroll
  for (int d = 1; d <= DM; ++d) {
    terms[d - 1] = ext_zero();
    const int t = T - d;
    if (t >= 0) {
      const int k = t + U;
      const int64_t pos = node_pos(p, b, k, U - diag_ulo(k, T));
      terms[d - 1] = ext_mul(xrec_get(p.ar, pos), wrec_get(wrec(p.wout, p, pos), NW, d - 1));
    }
  }
  const double lp = ext_log(ext_sum(terms));
  p.logpa[b] = lp;
  return lp;
}

// One direction of the lattice.  ALPHA: forward sweep with the incoming records;
// otherwise backward sweep with the node's outgoing records, beta of the terminal
// (t = T, u = U) seeded as 1 in the ring.  Moves that leave the lattice and moves with
// no source have zero weight, and sources outside the lattice have zero alpha, so no
// term needs a predicate; a node outside the lattice is forced to zero.  Out-of-range
// record reads return zero (buffer range check).  `prog` (LDS) receives the step index
// for the L2 warm-up waves.
template <int DM, int R, bool SW, bool ALPHA>
__device__ void sweep(const Params& p, int b, int T, int U, int tid, double* xm, int* xe, lds_int* prog) {
  constexpr int NW = 2 * DM + 1;
  constexpr int S = ring_size<DM>();
  constexpr int RWB = rec_bytes(DM);
  const int nsteps = T + U;
  const int WP = p.WP;
  const int64_t nrec = (int64_t)p.KD * WP;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((ALPHA ? p.win : p.wout) + b * nrec * RWB), (short)0, (int)(nrec * RWB), 0x00020000);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((ALPHA ? p.ar : p.br) + b * nrec * 16), (short)0, (int)(nrec * 16), 0x00020000);
  Ext h[R][S];
  Ext nb[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    nb[s] = ext_zero();
#pragma unroll
    for (int r = 0; r < R; ++r) h[r][s] = ext_zero();
  }
  if (!ALPHA) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (tid * R + r == U) h[r][S - 1] = ext_one();  // beta(T, U): the terminal
  }
  // NB record buffers, prefetched NB-1 steps ahead (NB divides the unroll length S)
  constexpr int NB = (DM <= 4 && R == 1) ? S : 3;
  WRec<DM> wb[NB][R];

  auto load_w = [&](int ks, WRec<DM> (&w)[R]) {
    const int k = ALPHA ? ks : nsteps - 1 - ks;
    const int base = k * WP - diag_ulo(k, T);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int off = (base + tid * R + r) * RWB;
      asm volatile("" : "+v"(off));  // keep the per-chunk constants in the instruction offset
      constexpr int NQ = WRec<DM>::NQ;
#pragma unroll
      for (int j = 0; j < NQ - 1; ++j) w[r].q[j] = __builtin_amdgcn_raw_buffer_load_b128(wr, off + 16 * j, 0, 0);
      // the record holds 12*NW bytes (NW odd): its last 16-byte word ends with 4 bytes of
      // padding, which are not loaded
      const u32x3v last = __builtin_amdgcn_raw_buffer_load_b96(wr, off + 16 * (NQ - 1), 0, 0);
      w[r].q[NQ - 1] = u32x4v{last.x, last.y, last.z, 0u};
    }
  };

#pragma unroll
  for (int j = 0; j < NB - 1; ++j) load_w(j, wb[j]);
  for (int k0 = 0; k0 < nsteps; k0 += S) {
#pragma unroll
    for (int ph = 0; ph < S; ++ph) {
      const int ks = k0 + ph;
      if (ks >= nsteps) break;
      // unconditional: past the last step the offsets fall outside the records of this
      // utterance and the buffer range check returns zeros (never consumed), and a
      // conditional load would make the wait before the next use cover this load too
      load_w(ks + NB - 1, wb[(ph + NB - 1) % NB]);
      const int k = ALPHA ? ks : nsteps - 1 - ks;
      const int base = k * WP - diag_ulo(k, T);
      Ext nv[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int u = tid * R + r, t = k - u;
        const bool act = (unsigned)t < (unsigned)T && u <= U;
        const WRec<DM>& w = wb[ph % NB][r];
        Ext terms[NW];
#pragma unroll
        for (int d = 1; d <= DM; ++d) terms[d - 1] = ext_mul(h[r][(ph - d + 4 * S) % S], w.get(d - 1));
        if (ALPHA) {
#pragma unroll
          for (int d = 0; d <= DM; ++d) {
            const Ext src = r > 0 ? h[r > 0 ? r - 1 : 0][(ph - 1 - d + 4 * S) % S] : nb[(ph - 1 - d + 4 * S) % S];
            terms[DM + d] = ext_mul(src, w.get(DM + d));
          }
        } else {
#pragma unroll
          for (int d = 0; d <= DM; ++d) {
            const Ext dst = r < R - 1 ? h[r < R - 1 ? r + 1 : 0][(ph - 1 - d + 4 * S) % S] : nb[(ph - 1 - d + 4 * S) % S];
            terms[DM + d] = ext_mul(dst, w.get(DM + d));
          }
        }
        Ext a = ext_sum_biased(terms);
        if (ALPHA && ks == 0 && u == 0) a = ext_one();
        if (!act) a = ext_zero();
        nv[r] = a;
        const int o = act ? (base + u) * 16 : -16;
        const uint64_t mb = __builtin_bit_cast(uint64_t, a.m);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4v{(uint32_t)mb, (uint32_t)(mb >> 32), (uint32_t)a.e, 0u}, xr, o, 0,
                                               0);
        if (!ALPHA && ks == nsteps - 1 && u == 0) beta_final(p, b, a);  // beta(0,0) = P
      }
#pragma unroll
      for (int r = 0; r < R; ++r) h[r][ph] = nv[r];
      nb[ph] = exchange<SW>(ALPHA ? nv[R - 1] : nv[0], ALPHA, ph & 1, xm, xe);
      if (SW) __hip_atomic_store(prog, ks, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  if (ALPHA && tid * R <= U && U < tid * R + R) (void)alpha_terminal<DM>(p, b, T, U);
}

// ------------------------------------------------------------------------------------
// Plain-float64 sweep (one wave, R label indices per lane).  Lane u keeps its values as
// plain float64 numbers x relative to a lane scale: value = x * 2^sc.  Every S steps
// each lane shifts its rings and sc so that its newest value is near 1; a neighbour's
// value arrives with the neighbour's scale and is converted once, so values of different
// labels on one anti-diagonal may lie any number of binary orders apart.  A step is then
// DM + (DM + 1) fused multiply-adds per label on plain numbers.  Every move weight of the
// utterance lies in [2^-300, 2^300] (checked by the node-weight kernel).  Mass lost to
// underflow (or an overflow) cannot be seen step by step without cost; it is caught
// afterwards by comparing log P from the two directions, each of which would lose a
// different share of it, and the caller then redoes both with the extended-range sweep.
// Alpha/beta records are written in extended form.
// Record buffers of the plain sweep, from {6, 3, 2}: as many as fit about 240 VGPRs (R
// labels of 2*DM+1 float64 per buffer) and keep the loads of NB-1 steps in flight within
// the 6-bit memory counter (per step: one load per slot pair and label, and R stores); 0
// when even 2 do not fit in 200 VGPRs (the extended-range sweep is used then).
template <int DM, int R>
__host__ __device__ constexpr int fast_buffers() {
  constexpr int NW = 2 * DM + 1;
  constexpr int per = R * 2 * NW;                        // VGPRs of one buffer
  constexpr int ops = slot_pairs(NW) * R + R;            // memory instructions per step
  constexpr int steps = 60 / ops;                        // steps in flight
  return (6 * per <= 240 && steps >= 5) ? 6
         : (3 * per <= 240 && steps >= 2) ? 3
         : (2 * per <= 200 && steps >= 1) ? 2 : 0;
}

// The NW weights of R consecutive labels, loaded slot by slot from the slot-major copy.
template <int DM, int R>
struct WPlain {
  static constexpr int NW = 2 * DM + 1;
  double v[NW][R];
};

template <int DM, int R, bool ALPHA>
__device__ void sweep_fast(const Params& p, int b, int T, int U, int lane, double* lp_out) {
  constexpr int S = ring_size<DM>();
  // weight buffers, prefetched NB-1 steps ahead
  constexpr int NB = fast_buffers<DM, R>();
  constexpr int UL = NB > S ? NB : S;  // steps unrolled per iteration
  static_assert(NB >= 2 && UL % S == 0 && UL % NB == 0, "unroll must hold whole rings and buffer rounds");
  const int nsteps = T + U;
  const int WP = p.WP, UW = p.UW;
  const int64_t nrec = (int64_t)p.KD * WP;
  const int64_t npw = (int64_t)p.KD * slot_pairs(p.NW) * UW * 2;  // plain weights of one utterance
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((ALPHA ? p.pwin : p.pwout) + b * npw), (short)0, (int)(npw * 8), 0x00020000);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((ALPHA ? p.ar : p.br) + b * nrec * 16), (short)0, (int)(nrec * 16), 0x00020000);
  const int u0 = lane * R;  // labels u0 .. u0 + R - 1 of this lane
  unsigned Tl[R];          // node (k - u, u) is in the lattice iff k - u < Tl
#pragma unroll
  for (int r = 0; r < R; ++r) Tl[r] = u0 + r <= U ? (unsigned)T : 0u;
  double h[R][S], nb[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    nb[s] = 0.0;
#pragma unroll
    for (int r = 0; r < R; ++r) h[r][s] = 0.0;
  }
  int sc = 0;             // the lane's scale: a value is x * 2^sc
  bool started = false;   // the lane holds a non-zero value, so its scale is fixed
  if (!ALPHA && u0 <= U && U < u0 + R) {  // beta(T, U): the terminal
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (u0 + r == U) h[r][S - 1] = 1.0;
    started = true;
  }
  WPlain<DM, R> wb[NB];
  auto load_w = [&](int ks, WPlain<DM, R>& w) {
    const int k = ALPHA ? ks : nsteps - 1 - ks;
    constexpr int NW = 2 * DM + 1, NP = slot_pairs(NW);
    int off = (k * NP * UW + lane) * 16;  // label u0 + r in column r * (UW / R) + lane
    asm volatile("" : "+v"(off));
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const u32x4v x = __builtin_amdgcn_raw_buffer_load_b128(wr, off + (pr * UW + r * (UW / R)) * 16, 0, 0);
        w.v[2 * pr][r] = __builtin_bit_cast(double, ((uint64_t)x.y << 32) | x.x);
        if (2 * pr + 1 < NW) w.v[2 * pr + 1][r] = __builtin_bit_cast(double, ((uint64_t)x.w << 32) | x.z);
      }
    }
  };
  // past the last step the loads fall outside this utterance's records (zeros) or hit
  // records that are never consumed; loading unconditionally keeps the wait counts of
  // the unrolled loop exact
#pragma unroll
  for (int j = 0; j < NB - 1; ++j) load_w(j, wb[j]);
  // whole blocks of UL steps: steps past the last diagonal are inactive for every lane
  for (int k0 = 0; k0 < nsteps; k0 += UL) {
#pragma unroll
    for (int q = 0; q < UL; ++q) {
      const int ph = q % S;  // ring slot
      if (ph == 0) {  // keep the lane's largest newest value near 1 (a zero lane shifts by 0)
        double big = fabs(h[0][S - 1]);
#pragma unroll
        for (int r = 1; r < R; ++r) big = fmax(big, fabs(h[r][S - 1]));
        int ex;
        (void)frexp(big, &ex);
        sc += ex;
#pragma unroll
        for (int s2 = 0; s2 < S; ++s2) {
          nb[s2] = ldexp(nb[s2], -ex);
#pragma unroll
          for (int r = 0; r < R; ++r) h[r][s2] = ldexp(h[r][s2], -ex);
        }
      }
      const int ks = k0 + q;
      load_w(ks + NB - 1, wb[(q + NB - 1) % NB]);
      const int k = ALPHA ? ks : nsteps - 1 - ks;
      const int base = k * WP - diag_ulo(k, T) + u0;
      double a[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const WPlain<DM, R>& w = wb[q % NB];
        // own moves (durations 1..DM), and the neighbour label's moves (durations 0..DM):
        // label u-1 (alpha) or u+1 (beta), in this lane or from the next lane over
        double c0 = 0.0, c1 = 0.0, c2 = 0.0, c3 = 0.0;
#pragma unroll
        for (int d = 1; d <= DM; ++d) {
          const double x = h[r][(ph - d + 4 * S) % S] * w.v[d - 1][r];
          if (d & 1) c0 += x; else c1 += x;
        }
#pragma unroll
        for (int d = 0; d <= DM; ++d) {
          const int sl = (ph - 1 - d + 4 * S) % S;
          const double src = ALPHA ? (r > 0 ? h[r > 0 ? r - 1 : 0][sl] : nb[sl])
                                   : (r < R - 1 ? h[r < R - 1 ? r + 1 : 0][sl] : nb[sl]);
          const double x = src * w.v[DM + d][r];
          if (d & 1) c3 += x; else c2 += x;
        }
        a[r] = (c0 + c1) + (c2 + c3);
        if (ALPHA && ks == 0 && u0 + r == 0) {  // alpha(0, 0)
          a[r] = 1.0;
          sc = 0;
          started = true;
        }
        if (!((unsigned)(k - u0 - r) < Tl[r])) a[r] = 0.0;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        h[r][ph] = a[r];
        int ea;
        const double ma = frexp(a[r], &ea);  // (0, 0) for a zero
        const int eo = a[r] != 0.0 ? ea + sc : kEZ;
        const int o = (unsigned)(k - u0 - r) < Tl[r] ? (base + r) * 16 : -16;
        const uint64_t mb = __builtin_bit_cast(uint64_t, ma);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4v{(uint32_t)mb, (uint32_t)(mb >> 32), (uint32_t)eo, 0u}, xr, o, 0,
                                               0);
        started = started || a[r] != 0.0;
      }
      // lane exchange: alpha passes its last label's value to the next lane, beta its
      // first label's value to the previous lane
      const double out = ALPHA ? a[R - 1] : a[0];
      const long long bits = __double_as_longlong(out);
      int lo = (int)(bits & 0xffffffffll), hi = (int)(bits >> 32), e = sc;
      constexpr int ctl = ALPHA ? 0x138 : 0x130;  // wave_shr:1 / wave_shl:1
      lo = __builtin_amdgcn_update_dpp(0, lo, ctl, 0xf, 0xf, false);
      hi = __builtin_amdgcn_update_dpp(0, hi, ctl, 0xf, 0xf, false);
      e = __builtin_amdgcn_update_dpp(0, e, ctl, 0xf, 0xf, false);
      const double m = __longlong_as_double(((long long)(unsigned)hi << 32) | (unsigned)lo);
      {  // an empty lane takes a scale that puts its first input near 1 (the sender's
         // own scale may be stale at the wavefront, far from the value it sends)
        int em;
        (void)frexp(m, &em);  // 0 for a zero
        if (!started) sc = e + em;
      }
      started = started || m != 0.0;
      nb[ph] = ldexp(m, e - sc);  // into this lane's scale
    }
  }
  if (ALPHA) {
    if (u0 <= U && U < u0 + R) *lp_out = alpha_terminal<DM>(p, b, T, U);
  } else if (lane == 0) {  // beta(0,0) = P: the value of the last step, still in the ring
    const int last = (nsteps - 1) % S;
    double a = h[0][0];
#pragma unroll
    for (int s2 = 1; s2 < S; ++s2)
      if (s2 == last) a = h[0][s2];
    int ea;
    const double ma = frexp(a, &ea);
    const Ext P = a != 0.0 ? Ext{ma, ea + sc} : ext_zero();
    beta_final(p, b, P);
    *lp_out = ext_log(P);
  }
}

// Plain-float64 sweep over several waves (U1max > 256): the lanes of all waves of the
// work-group run across the labels, R per lane, with the lane scales, renormalisation and
// per-step arithmetic of the single-wave sweep; the neighbour's value goes through LDS
// with one barrier per step, and the records of the next step are loaded while that
// exchange runs.  Alpha and beta run in different work-groups here, so the log P
// comparison is not available: each lane checks instead that every value it creates,
// converts or shifts stays within [2^-700, 2^700] (then, with every weight in
// [2^-300, 2^300], no product or sum can underflow or overflow), and the work-group redoes
// the direction with the extended-range sweep when any lane saw a value outside it.
template <int DM, int R>
__host__ __device__ constexpr bool fast_mw_ok() {
  return R * 2 * (2 * DM + 1) + 2 * (R + 1) * ring_size<DM>() <= 150;  // VGPRs at 768 threads
}

__device__ __forceinline__ bool out_of_range(double x) {  // non-zero and outside [2^-700, 2^700]
  const double a = fabs(x);
  return a != 0.0 && (a < 0x1p-700 || a > 0x1p700);
}

template <int DM, int R, bool ALPHA>
__device__ bool sweep_fast_mw(const Params& p, int b, int T, int U, int tid, double* xm, int* xe) {
  constexpr int S = ring_size<DM>();
  const int nt = blockDim.x;
  const int nsteps = T + U;
  const int WP = p.WP, UW = p.UW;
  const int64_t nrec = (int64_t)p.KD * WP;
  const int64_t npw = (int64_t)p.KD * slot_pairs(p.NW) * UW * 2;  // plain weights of one utterance
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((ALPHA ? p.pwin : p.pwout) + b * npw), (short)0, (int)(npw * 8), 0x00020000);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((ALPHA ? p.ar : p.br) + b * nrec * 16), (short)0, (int)(nrec * 16), 0x00020000);
  const int u0 = tid * R;
  unsigned Tl[R];
#pragma unroll
  for (int r = 0; r < R; ++r) Tl[r] = u0 + r <= U ? (unsigned)T : 0u;
  double h[R][S], nb[S];
#pragma unroll
  for (int s2 = 0; s2 < S; ++s2) {
    nb[s2] = 0.0;
#pragma unroll
    for (int r = 0; r < R; ++r) h[r][s2] = 0.0;
  }
  int sc = 0;
  bool started = false, trouble = false;
  if (!ALPHA && u0 <= U && U < u0 + R) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (u0 + r == U) h[r][S - 1] = 1.0;
    started = true;
  }
  WPlain<DM, R> w;  // the slot-pair-major plain weights of this lane's labels
  auto load_w = [&](int ks) {
    const int k = ALPHA ? ks : nsteps - 1 - ks;
    constexpr int NW = 2 * DM + 1, NP = slot_pairs(NW);
    const int off = (k * NP * UW + tid) * 16;  // label u0 + r in column r * (UW / R) + tid
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const u32x4v x = __builtin_amdgcn_raw_buffer_load_b128(wr, off + (pr * UW + r * (UW / R)) * 16, 0, 0);
        w.v[2 * pr][r] = __builtin_bit_cast(double, ((uint64_t)x.y << 32) | x.x);
        if (2 * pr + 1 < NW) w.v[2 * pr + 1][r] = __builtin_bit_cast(double, ((uint64_t)x.w << 32) | x.z);
      }
    }
  };
  load_w(0);
  for (int k0 = 0; k0 < nsteps; k0 += S) {
#pragma unroll
    for (int ph = 0; ph < S; ++ph) {
      if (ph == 0) {  // keep the lane's largest newest value near 1
        double big = fabs(h[0][S - 1]);
#pragma unroll
        for (int r = 1; r < R; ++r) big = fmax(big, fabs(h[r][S - 1]));
        int ex;
        (void)frexp(big, &ex);
        sc += ex;
#pragma unroll
        for (int s2 = 0; s2 < S; ++s2) {
          nb[s2] = ldexp(nb[s2], -ex);
          trouble |= out_of_range(nb[s2]);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            h[r][s2] = ldexp(h[r][s2], -ex);
            trouble |= out_of_range(h[r][s2]);
          }
        }
      }
      const int ks = k0 + ph;
      const int k = ALPHA ? ks : nsteps - 1 - ks;
      const int base = k * WP - diag_ulo(k, T) + u0;
      double a[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        double c0 = 0.0, c1 = 0.0, c2 = 0.0, c3 = 0.0;
#pragma unroll
        for (int d = 1; d <= DM; ++d) {
          const double x = h[r][(ph - d + 4 * S) % S] * w.v[d - 1][r];
          if (d & 1) c0 += x; else c1 += x;
        }
#pragma unroll
        for (int d = 0; d <= DM; ++d) {
          const int sl = (ph - 1 - d + 4 * S) % S;
          const double src = ALPHA ? (r > 0 ? h[r > 0 ? r - 1 : 0][sl] : nb[sl])
                                   : (r < R - 1 ? h[r < R - 1 ? r + 1 : 0][sl] : nb[sl]);
          const double x = src * w.v[DM + d][r];
          if (d & 1) c3 += x; else c2 += x;
        }
        a[r] = (c0 + c1) + (c2 + c3);
        if (ALPHA && ks == 0 && u0 + r == 0) {
          a[r] = 1.0;
          sc = 0;
          started = true;
        }
        if (!((unsigned)(k - u0 - r) < Tl[r])) a[r] = 0.0;
        trouble |= out_of_range(a[r]);
      }
      // the records of the next step, during the exchange (unconditional: past the last
      // step the offsets fall outside this utterance's records and read zeros)
      load_w(ks + 1);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        h[r][ph] = a[r];
        int ea;
        const double ma = frexp(a[r], &ea);
        const int eo = a[r] != 0.0 ? ea + sc : kEZ;
        const int o = (unsigned)(k - u0 - r) < Tl[r] ? (base + r) * 16 : -16;
        const uint64_t mb = __builtin_bit_cast(uint64_t, ma);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4v{(uint32_t)mb, (uint32_t)(mb >> 32), (uint32_t)eo, 0u}, xr, o, 0,
                                               0);
        started = started || a[r] != 0.0;
      }
      // neighbour exchange through LDS
      const int par = (ks & 1) * 1024;
      xm[par + tid] = ALPHA ? a[R - 1] : a[0];
      xe[par + tid] = sc;
      // barrier on the LDS exchange only: __syncthreads() would also wait for every
      // outstanding global load, including the prefetches of later steps
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const int src = ALPHA ? tid - 1 : tid + 1;
      const bool has = src >= 0 && src < nt;
      const double m = has ? xm[par + src] : 0.0;
      const int e = has ? xe[par + src] : 0;
      {  // an empty lane takes a scale that puts its first input near 1 (the sender's
         // own scale may be stale at the wavefront, far from the value it sends)
        int em;
        (void)frexp(m, &em);  // 0 for a zero
        if (!started) sc = e + em;
      }
      started = started || m != 0.0;
      nb[ph] = ldexp(m, e - sc);
      trouble |= m != 0.0 && out_of_range(nb[ph]);
    }
  }
  trouble = __syncthreads_or(trouble);
  if (trouble) return true;
  if (ALPHA) {
    if (u0 <= U && U < u0 + R) (void)alpha_terminal<DM>(p, b, T, U);
  } else if (tid == 0) {
    const int last = (nsteps - 1) % S;
    double a = h[0][0];
#pragma unroll
    for (int s2 = 1; s2 < S; ++s2)
      if (s2 == last) a = h[0][s2];
    int ea;
    const double ma = frexp(a, &ea);
    beta_final(p, b, a != 0.0 ? Ext{ma, ea + sc} : ext_zero());
  }
  return false;
}

// L2 warm-up for a single-wave sweep: a helper wave touches every 128-byte line of the
// weight records of the diagonals its chain will reach next, at most kLead diagonals
// ahead of it (the chain never waits for it).  Loads for kBatch diagonals are issued
// before any is consumed, so the helper advances kBatch diagonals per memory round trip
// rather than one.
constexpr int kLead = 64;
constexpr int kBatch = 16;

__device__ void l2_warm(const Params& p, int b, int nsteps, bool alpha, int lane, lds_int* prog) {
  const int64_t dbytes = (int64_t)p.WP * p.RW;  // one diagonal of records
  const int lines = (int)((dbytes + 127) / 128);
  const char* base = (alpha ? p.win : p.wout) + (int64_t)b * p.KD * dbytes;
  uint32_t acc = 0;
  for (int ks0 = 0; ks0 < nsteps; ks0 += kBatch) {
    while (ks0 + kBatch - 1 > __hip_atomic_load(prog, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) + kLead)
      __builtin_amdgcn_s_sleep(2);
    for (int l = lane; l < lines; l += kWave) {
      uint32_t x[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int ks = ks0 + j < nsteps ? ks0 + j : nsteps - 1;
        const int k = alpha ? ks : nsteps - 1 - ks;
        x[j] = *(const uint32_t*)(base + (int64_t)k * dbytes + (int64_t)l * 128);
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) acc += x[j];
    }
  }
  if (acc == 0x9e3779b9u && p.B < 0) p.uok[0] = (int)acc;  // keeps the touching loads alive
}

// Lattice kernel, one work-group per (utterance, direction).  SW (U1max <= 256): 128
// threads, wave 0 the chain; the plain-float64 sweep where its registers fit
// (fast_buffers), checked by the agreement of log P from the two directions, and the
// extended-range sweep (wave 1 keeping its records warm in L2) otherwise or when the
// check fails.  Longer label sequences: up to 768 threads (1024 for R = 8) with the
// range-checked multi-wave plain sweep where its registers fit (fast_mw_ok) and the
// extended-range sweep after it or instead of it.
template <int DM, int R, bool SW>
__global__ __launch_bounds__(SW ? 128 : (R <= 4 ? 768 : 1024)) void k_lattice(const Params p) {
  __shared__ double xm[SW ? 1 : 2 * 1024];
  __shared__ int xe[SW ? 1 : 2 * 1024];
  __shared__ unsigned long long s_sumU;
  __shared__ int s_prog[2];
  __shared__ double s_lp[2];
  __shared__ int s_redo;
  const int b = blockIdx.x >> 1;
  const int dir = blockIdx.x & 1;  // 0: alpha, 1: beta
  const bool alpha_side = dir == 0, beta_side = dir == 1;
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
  if (tid == 0) {
    s_sumU = 0;
    s_prog[0] = s_prog[1] = -1;
  }
  if (__syncthreads_or(bad)) status |= 4;
  if (beta_side && p.red == 4) {
    unsigned long long part = 0;
    for (int bb = tid; bb < p.Btot; bb += nt) part += (unsigned long long)p.Ulen_tot[bb];
    if (part) atomicAdd(&s_sumU, part);
  }
  __syncthreads();
  if (beta_side && tid == 0) p.wts[b] = reduction_weight(p, b, (int64_t)s_sumU);
  const int T = (int)T64, U = (int)U64;
  if (status != 0 || T == 0) {
    if (tid == 0) {
      if (beta_side) {
        p.logp[b] = status ? __builtin_nan("") : -__builtin_inf();
        p.pm[b] = 0.0;
        p.pe[b] = kEZ;
        p.uok[b] = 0;
        if (p.ustatus) p.ustatus[b] = status ? status : 8;
      }
      if (alpha_side) p.logpa[b] = status ? __builtin_nan("") : -__builtin_inf();
    }
    return;
  }
  if constexpr (SW) {
    // one direction per work-group: wave 0 runs the chain, wave 1 keeps the records of
    // the extended-range sweep warm in L2
    const int wv = tid >> 6, lane = tid & (kWave - 1);
    lds_int* prog = (lds_int*)&s_prog[0];
    if constexpr (fast_buffers<DM, R>() > 0) {
      if (!p.xflag[b] && p.pwin) {
        if (wv == 0) {
          if (alpha_side) sweep_fast<DM, R, true>(p, b, T, U, lane, &s_lp[0]);
          else sweep_fast<DM, R, false>(p, b, T, U, lane, &s_lp[0]);
        }
        __syncthreads();
        // The direction that finishes second compares the two log P values (both sum
        // the same probability mass; rounding alone stays below 1e-12) and, unless both
        // are finite and differ by at most 1e-9, redoes both directions with the
        // extended-range sweep: mass lost to underflow differs between the directions, and
        // when it is all of it both read -inf, which only the extended sweep can tell
        // from an utterance without alignments.  The counter was zeroed by the
        // row-statistics pass of this call.
        if (tid == 0) {
          __hip_atomic_store(p.lpx + 2 * b + dir, s_lp[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const int old = __hip_atomic_fetch_add(p.lcnt + b, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
          int redo = 0;
          if (old == 1) {
            const double other =
                __hip_atomic_load(p.lpx + 2 * b + (dir ^ 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const double mine = s_lp[0];
            redo = (isfinite(mine) && isfinite(other) && fabs(mine - other) <= 1e-9) ? 0 : 1;
          }
          s_redo = redo;
        }
        __syncthreads();
        if (!s_redo) return;
        for (int pass = 0; pass < 2; ++pass) {
          if (tid == 0) s_prog[0] = -1;
          __syncthreads();
          if (wv == 0) {
            if (pass == 0) sweep<DM, R, true, true>(p, b, T, U, lane, xm, xe, prog);
            else sweep<DM, R, true, false>(p, b, T, U, lane, xm, xe, prog);
          } else {
            l2_warm(p, b, T + U, pass == 0, lane, prog);
          }
          __syncthreads();
        }
        return;
      }
    }
    if (wv == 0) {
      if (alpha_side) sweep<DM, R, true, true>(p, b, T, U, lane, xm, xe, prog);
      else sweep<DM, R, true, false>(p, b, T, U, lane, xm, xe, prog);
    } else {
      l2_warm(p, b, T + U, alpha_side, lane, prog);
    }
  } else {
    if constexpr (fast_mw_ok<DM, R>()) {
      if (!p.xflag[b] && p.pwin) {
        const bool trouble = dir == 0 ? sweep_fast_mw<DM, R, true>(p, b, T, U, tid, xm, xe)
                                      : sweep_fast_mw<DM, R, false>(p, b, T, U, tid, xm, xe);
        if (!trouble) return;
        __syncthreads();  // the exchange arrays are reused below
      }
    }
    if (dir == 0)
      sweep<DM, R, false, true>(p, b, T, U, tid, xm, xe, (lds_int*)&s_prog[0]);
    else
      sweep<DM, R, false, false>(p, b, T, U, tid, xm, xe, (lds_int*)&s_prog[0]);
  }
}

// ------------------------------------------------------------------------------------
// Posteriors and the per-node record of the gradient pass:
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

// A group of NG lanes works on one node (as in the node weights): lane d handles the
// blank and the label move of duration value d; the group sums give O, c_blank, c_label.
// The first work-group also reduces the loss (the lattice has finished every log P) unless
// the call writes no loss.  An upstream gradient (chain rule) scales w_b.
template <int DM>
__global__ __launch_bounds__(256) void k_coef(const Params p) {
  constexpr int NW = 2 * DM + 1;
  constexpr int NG = DM < 8 ? 8 : (DM < 16 ? 16 : 32);
  if (p.loss && blockIdx.x == 0 && threadIdx.x == 0) reduce_loss(p);
  const int64_t gt = (int64_t)xcd_block(blockIdx.x, gridDim.x) * 256 + threadIdx.x;
  const int j = threadIdx.x & (NG - 1);
  const int64_t g = gt / NG;
  const int64_t per = (int64_t)p.KD * p.WP;
  const int b = (int)(g / per);
  // whole groups leave together below: every condition depends on the position only
  if (b >= p.B) return;
  // the three per-utterance words in one round trip (an ok utterance has valid lengths)
  const int ok = p.uok[b];
  const int T = (int)p.Tlen[b], U = (int)p.Ulen[b];
  if (!ok) return;
  const int64_t rem = g - (int64_t)b * per;
  const int k = (int)(rem / p.WP);
  const int i = (int)(rem - (int64_t)k * p.WP);
  if (k >= T + U) return;
  const int u = diag_ulo(k, T) + i;
  if (u > min(k, U)) return;
  const int t = k - u;
  const int64_t pos = node_pos(p, b, k, i);

  const Ext a = xrec_get(p.ar, pos);
  const char* wr = wrec(p.wout, p, pos);
  const double Pm = p.pm[b];
  const int Pe = p.pe[b];
  const int d = j;
  double gb = 0.0, gy = 0.0;  // posteriors of the blank / label move of duration d
  if (d <= DM) {
    if (d >= 1) {
      Ext bt = ext_zero();
      if (t + d < T) {
        const int k2 = k + d;
        bt = xrec_get(p.br, node_pos(p, b, k2, u - diag_ulo(k2, T)));
      } else if (t + d == T && u == U) {
        bt = ext_one();
      }
      const Ext gm = ext_mul(ext_mul(a, wrec_get(wr, NW, d - 1)), bt);
      gb = ext_to_double(Ext{gm.m / Pm, gm.e - Pe});
    }
    if (u < U && t + d < T) {
      const int k2 = k + d + 1;
      const Ext bt = xrec_get(p.br, node_pos(p, b, k2, u + 1 - diag_ulo(k2, T)));
      const Ext gm = ext_mul(ext_mul(a, wrec_get(wr, NW, DM + d)), bt);
      gy = ext_to_double(Ext{gm.m / Pm, gm.e - Pe});
    }
  }
  double cb = gb, cl = gy;
#pragma unroll
  for (int o = NG / 2; o >= 1; o >>= 1) {
    cb += __shfl_xor(cb, o, NG);
    cl += __shfl_xor(cl, o, NG);
  }
  const double O = cb + cl;
  const double wgt = p.gscale ? p.wts[b] * (double)p.gscale[p.red == 0 ? b : 0] : p.wts[b];
  const double* pr = p.pr + pos * p.NPR;
  float* rec = p.rec + pos * p.RS;
  if (j == 0) {
    const float4 rs = p.rstat[pos];
    int y = -1;
    if (u < U) y = (int)p.labels[(int64_t)b * p.lab_stride + u];
    double Gb = wgt * (O * pr[0] - cb);
    const double Gy = wgt * (O * pr[1] - cl);
    if (y == p.blank) {  // both corrections land on the blank column
      Gb -= wgt * cl;
      y = -1;
    }
    const double wO = wgt * O;
    if (p.dtype == 0) {  // A = w O 2^-K and the row maximum
      rec[0] = (float)(wO * exp2(-(double)rs.y));
      rec[1] = rs.x;
    } else {  // the sign of w O and C = c + K - log2|w O| (base 2)
      rec[0] = wO < 0.0 ? -1.f : 1.f;
      rec[1] = (float)((double)rs.x + (double)rs.y - log2(fabs(wO)));
    }
    rec[2] = (float)Gb;
    rec[3] = (float)Gy;
    rec[4] = __int_as_float(y);
  }
  if (d <= DM) {
    const int idx = p.didx[d];
    if (idx >= 0) rec[5 + idx] = (float)(wgt * (O * pr[2 + d] - (gb + gy)));
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
  const dim3 grid(2 * p.B);  // one work-group per (utterance, direction)
  if (u1 <= 64) {
    hipLaunchKernelGGL((k_lattice<DM, 1, true>), grid, dim3(128), 0, st, p);
  } else if (u1 <= 128) {
    hipLaunchKernelGGL((k_lattice<DM, 2, true>), grid, dim3(128), 0, st, p);
  } else if (u1 <= 256) {
    hipLaunchKernelGGL((k_lattice<DM, 4, true>), grid, dim3(128), 0, st, p);
  } else {
    // at most 768 threads for R <= 4 (about 170 VGPRs per lane), 1024 for R = 8
    int R = u1 <= 768 ? 1 : u1 <= 1536 ? 2 : u1 <= 3072 ? 4 : 8;
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
    case 0: {  // node weights: NG lanes per position
      const int ng = p.DM < 8 ? 8 : (p.DM < 16 ? 16 : 32);
      const dim3 gridw((unsigned)((n * ng + 255) / 256));
      if (p.DM == 4) hipLaunchKernelGGL((k_node_weights<4>), gridw, dim3(256), 0, st, p);
      else if (p.DM == 8) hipLaunchKernelGGL((k_node_weights<8>), gridw, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((k_node_weights<16>), gridw, dim3(256), 0, st, p);
      return hipGetLastError();
    }
    case 1:  // lattice
      if (p.DM == 4) return launch_lattice_dm<4>(p, st);
      if (p.DM == 8) return launch_lattice_dm<8>(p, st);
      return launch_lattice_dm<16>(p, st);
    case 2: {  // coefficients (and the loss reduction): NG lanes per position
      const int ng = p.DM < 8 ? 8 : (p.DM < 16 ? 16 : 32);
      const dim3 gridc((unsigned)((n * ng + 255) / 256));
      if (p.DM == 4) hipLaunchKernelGGL((k_coef<4>), gridc, dim3(256), 0, st, p);
      else if (p.DM == 8) hipLaunchKernelGGL((k_coef<8>), gridc, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((k_coef<16>), gridc, dim3(256), 0, st, p);
      return hipGetLastError();
    }
    default:  // loss reduction over the whole batch
      hipLaunchKernelGGL(k_reduce, dim3(1), dim3(64), 0, st, p);
      return hipGetLastError();
  }
}

}  // namespace tdt
