// Lattice side of the TDT loss on gfx950:
//   node weights  — duration log-softmax, the log-domain move ingredients and the plain
//                   float64 weight of every move out of a node (one group of lanes per
//                   node, lane d = duration value d);
//   lattice tiles — float64 alpha and beta sweeps over the T x (U+1) lattice (the
//                   alpha/beta passes of the page "tdt-loss: add TDT loss kernel", comment
//                   "What's in it": float64, no 1024-label limit), as an anti-diagonal
//                   wavefront with the label index across the lanes of one wave; up to
//                   256 labels the waves of one work-group sweep 64-label tiles at once,
//                   linked through LDS; longer label sequences are cut into tiles of 64
//                   labels x 48 frames swept band after band (one launch per band of
//                   tiles), so there is no limit on the label count and no work-group
//                   waits for another;
//   coefficients  — posteriors of the moves out of each node and the per-node record of
//                   the gradient pass, plus the loss reduction.
//
// Probabilities are kept in the linear domain: plain float64 numbers relative to a
// per-lane binary scale where every move weight lies in [2^-300, 2^300] (range-checked
// step by step), extended-range float64 (mantissa and a separate int exponent) otherwise,
// so a lattice step is multiply-adds and exponent arithmetic with no exp/log on the
// serial chain of the plain sweep.
#include "tdt_kernels.h"

namespace tdt {

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// A buffer offset beyond every buffer range used here (all below 2^31 bytes): loads at
// it read zeros and stores to it are dropped.
constexpr int kBadOff = (int)0x80000000u;

// Reduction weight w_b of utterance b (d reduced loss / d loss_b).
__device__ double reduction_weight(const Params& p, int b, int64_t sumU) {
  switch (p.red) {
    case 3: return 1.0 / (double)p.B;  // mean_batch
    case 2: {                          // mean
      const int64_t U = p.Ulen[b];
      return 1.0 / ((double)p.B * (double)(U > 1 ? U : 1));
    }
    case 4: return 1.0 / (double)(sumU > 1 ? sumU : 1);  // mean_volume
    default: return 1.0;                                 // none, sum
  }
}

// ------------------------------------------------------------------------------------
// Node weights: for node n = (t,u) of utterance b
//   lb = l_blank - sigma, ly = l_label - sigma (l = log-softmax of the token logits),
//   lambda_i = log-softmax of the duration logits,
//   W_blank(d) = exp(lb + lambda_d)  (d > 0; t+d < T, or t+d = T at u = U),
//   W_label(d) = exp(ly + lambda_d)  (u < U, t+d < T),
// stored as the log-domain ingredients (lb, ly, lambda) and as plain float64 weights by
// slot pairs (zero for absent durations and for moves that leave the lattice).  One lane
// per position of the padded box, the grid [box / 256, utterances] (blockIdx.y, strided
// by gridDim.y, picks the utterance), so a wave writes 64 consecutive records.  A plain
// weight is computed as exp(lb) softmax(g)_d, the same number as exp(lb + lambda_d) up to
// rounding, so a node takes D + 2 exponentials.  The lane also combines the row
// segments' log-sum-exp partials into the row statistics (c, K), and reads the node's
// blank and label logits from the token view.
template <int DM>
__global__ __launch_bounds__(256) void k_node_weights(const Params p) {
  if (p.xns && blockIdx.x == 0 && blockIdx.y == 0) {
    // the linked columns' control words and link progress (nothing written yet)
    for (int i = threadIdx.x; i < 2 * p.B; i += 256) p.xctl[i] = XCtl{0, 0, 0, 0, 0.0};
    for (int i = threadIdx.x; i < 2 * p.B * p.nU; i += 256) p.xprod[i] = -(1 << 30);
  }
  const int q = (int)(blockIdx.x * 256 + threadIdx.x);
  if (q >= p.box) return;
  int k, i;
  box_pos(p, q, k, i);
  const int u = diag_ulo(p, k) + i, t = k - u;
  const bool base2 = p.dtype != 0;
  const float F = base2 ? 1.f : kLog2e;
  constexpr double kLo = -300.0 * 0.6931471805599453, kHi = 300.0 * 0.6931471805599453;
  for (int b = blockIdx.y; b < p.B; b += gridDim.y) {
    const int64_t T64 = p.Tlen[b], U64 = p.Ulen[b];
    if (!utt_dims_ok(p, T64, U64)) continue;
    const int T = (int)T64, U = (int)U64;
    if (t >= T || u > U) continue;
    const int64_t pos = (int64_t)b * p.box + q;

    // the blank and label logits of the node (the label read first: its column is data)
    const int64_t tbase = (int64_t)b * p.ts0 + (int64_t)t * p.ts1 + (int64_t)u * p.ts2;
    const int64_t yy = u < U ? p.labels[(int64_t)b * p.lab_stride + u] : -1;
    const float hb = load_tok(p, tbase + p.blank);
    // duration logits by duration value (absent values: -inf)
    const int64_t dbase = (int64_t)b * p.ds0 + (int64_t)t * p.ds1 + (int64_t)u * p.ds2;
    double gv[DM + 1];
    double gmax = -__builtin_inf();
#pragma unroll
    for (int d = 0; d <= DM; ++d) {
      const int idx = p.didx[d];
      gv[d] = idx >= 0 ? (double)load_dur(p, dbase + idx) : -__builtin_inf();
      gmax = fmax(gmax, gv[d]);
    }

    // log-sum-exp of the token logits from the row-segment partials; 16-bit logits keep
    // their shifts in base-2 units (see k_row_partial).  Each float32 partial sum is
    // rescaled to the common shift in float32 and summed in float64.  A NaN partial
    // (logits beyond the float range of the shift) propagates.
    const float* part = p.part + (((int64_t)b * p.Tmax + t) * p.U1max + u) * 2 * p.nseg;  // node-major
    float mx = -__builtin_inff();
    for (int s2 = 0; s2 < p.nseg; ++s2)
      if (!(part[2 * s2 + 1] <= 0.f)) mx = fmaxf(mx, part[2 * s2]);
    double S = 0.0;
    for (int s2 = 0; s2 < p.nseg; ++s2) {
      const float m2 = part[2 * s2], p2 = part[2 * s2 + 1];
      if (!(p2 <= 0.f)) S += (double)(p2 * __builtin_amdgcn_exp2f((m2 - mx) * F));
    }
    const double K = log2(S);
    const double L = row_lse(base2, (double)mx, K);  // natural-log normaliser
    // a label outside [0, V) is a data error the lattice reports; its move is impossible
    const float hy = (yy >= 0 && yy < p.V) ? load_tok(p, tbase + yy) : -__builtin_inff();
    const double lb = (double)hb - L - p.sigma;
    const double ly = hy > -__builtin_inff() ? (double)hy - L - p.sigma : -__builtin_inf();
    p.stat[pos] = make_float2(mx, (float)K);

    // duration log-softmax: lambda_d = g_d - gmax - log(sum exp(g - gmax))
    double e[DM + 1];
    double sg = 0.0;
#pragma unroll
    for (int d = 0; d <= DM; ++d) {
      e[d] = p.didx[d] >= 0 ? exp(gv[d] - gmax) : 0.0;
      sg += e[d];
    }
    const double lsg = log(sg), rsg = 1.0 / sg;
    const double eb = exp(lb), ey = exp(ly);

    double* lg = p.lg + pos * p.LG;
    lg[0] = lb;
    lg[1] = ly;
    // plain outgoing weights; a non-zero weight outside [2^-300, 2^300] (or an exp(lb),
    // exp(ly) above 2^300, whose product form could overflow) sends the utterance to the
    // extended-range sweeps
    bool wide = lb > kHi || ly > kHi;
    const int len = diag_len(p, k);
    double* pw = p.pw ? p.pw + ((int64_t)b * pw_utt_entries(p.NP, p.box, p.KD) +
                                (int64_t)p.NP * (q - i + 3 * (int64_t)k) + pw_col(i, len, p.R)) * 2
                      : nullptr;
    const int64_t pstride = (int64_t)(len + 3) * 2;  // doubles between slot pairs
#pragma unroll
    for (int d = 0; d <= DM; ++d) {
      const int idx = p.didx[d];
      const bool has = idx >= 0;
      const double lam = gv[d] - gmax - lsg;
      if (has) lg[2 + idx] = lam;
      const double sm = e[d] * rsg;  // softmax(g)_d
      if (d >= 1) {
        const bool ok = has && (t + d < T || (t + d == T && u == U));
        const double x = ok ? lb + lam : -__builtin_inf();
        wide |= x > -__builtin_inf() && (x < kLo || x > kHi);
        const int s = d - 1;
        if (pw) pw[(s >> 1) * pstride + (s & 1)] = ok ? eb * sm : 0.0;
      }
      const bool okl = has && u < U && t + d < T;
      const double xl = okl ? ly + lam : -__builtin_inf();
      wide |= xl > -__builtin_inf() && (xl < kLo || xl > kHi);
      const int s = DM + d;
      if (pw) pw[(s >> 1) * pstride + (s & 1)] = okl ? ey * sm : 0.0;
    }
    if (wide) atomicOr(p.xflag + b, 1);
  }
}

// ------------------------------------------------------------------------------------
// Lattice tiles.
//
// A tile covers frames [t0, t1) and labels [u0, ulast] of one utterance; lane l of the
// sweeping wave owns labels u0 + l R .. u0 + l R + R - 1.  Step by step the wave walks the
// tile's anti-diagonals k = t + u.  Values of nodes outside the tile that the tile
// needs come from memory: the alpha (beta) of up to DM frames below (above) the tile,
// replayed as if computed, and, for alpha, the label moves entering the tile's first
// label from the tile to its left (`lx`, written by that tile); for beta the last lane
// reads the beta of the label right of the tile.  Those tiles belong to earlier bands.
//
// Alpha runs in push form: when node (t, u) is done, its value times each of its outgoing
// weights is added to accumulator rings for the destinations (blank: (t+d, u) in the same
// label; label: (t+d, u+1)), and the complete label contribution into (t, u+1) moves to
// the next label (same lane, or the next lane by a DPP shift) for the next step.  Beta
// runs in pull form from the beta of the destinations.  Both read only the node's own
// outgoing weight record, which lies on the node's own diagonal: the records a step reads
// are contiguous.
struct Tile {
  int b, T, U;
  int t0, t1;       // frames of the tile: [t0, t1), t1 <= T
  int u0, ulast;    // labels: [u0, ulast], ulast <= U
  bool below, above, left, right;  // other tiles hold frames < t0, frames >= t1, labels < u0, labels > ulast
};

__device__ __forceinline__ bool make_tile(const Params& p, int b, int T, int U, int i, int j, int width,
                                          Tile& tl) {
  tl.b = b;
  tl.T = T;
  tl.U = U;
  tl.t0 = i * p.TT;
  tl.t1 = min(tl.t0 + p.TT, T);
  tl.u0 = j * width;
  tl.ulast = min(tl.u0 + width - 1, U);
  tl.below = tl.t0 > 0;
  tl.above = tl.t1 < T;
  tl.left = tl.u0 > 0;
  tl.right = tl.ulast < U;
  return tl.t0 < T && tl.u0 <= U;
}

// Ring slots: S >= DM + 2 (the accumulators of DM + 1 future frames plus the contribution
// in flight to the next label), a multiple of 6 so that unrolled loops hold whole rings
// and whole rounds of the prefetch buffers.
template <int DM>
__host__ __device__ constexpr int ring_size() { return ((DM + 2 + 5) / 6) * 6; }

// Prefetch buffers of the plain sweeps: as many as fit about 200 VGPRs together with the
// alpha rings (2 R S float64) and keep the loads of NB - 1 steps within the 6-bit memory
// counter; NB divides the ring size.  0: no plain sweep (durations beyond 8 run the
// extended-range sweeps only).
template <int DM, int R>
__host__ __device__ constexpr int plain_buffers() {
  constexpr int NP = DM + 1, S = ring_size<DM>();
  constexpr int budget = 200 - 4 * R * S;
  constexpr int per = 4 * NP * R + 8;      // VGPRs of one buffer (weights and boundary records)
  constexpr int mem = NP * R + 4;          // memory instructions per step
  constexpr int steps = 56 / mem;          // steps in flight the counter allows
  return (6 * per <= budget && steps >= 5) ? 6
         : (S % 4 == 0 && 4 * per <= budget && steps >= 3) ? 4
         : (3 * per <= budget && steps >= 2) ? 3
         : (2 * per <= budget && steps >= 1) ? 2 : 0;
}

// Range check of the plain sweeps by binary exponents (frexp: x = m 2^e, m in [0.5, 1);
// e = 0 for a zero): a value that left [2^-700, 2^700], or an input that would have
// entered the lane's scale outside it, sends the tile to the extended-range sweep.
struct RangeTrack {
  int lo = 0, hi = 0;
  __device__ __forceinline__ void add_exp(int e) {
    lo = min(lo, e);
    hi = max(hi, e);
  }
  __device__ __forceinline__ void add(double x) { add_exp(__builtin_amdgcn_frexp_exp(x)); }
  __device__ __forceinline__ bool bad() const { return lo <= -700 || hi > 700; }
};

// An extended record (float64 value, int32 binary exponent) as the 16 bytes of a buffer
// load, normalised (a zero gets the extended zero's exponent).
__device__ __forceinline__ Ext rec_ext(u32x4v x) {
  return ext_norm(__builtin_bit_cast(double, ((uint64_t)x.y << 32) | x.x), (int)x.z);
}
__device__ __forceinline__ u32x4v ext_rec(Ext v) {
  const uint64_t mb = __builtin_bit_cast(uint64_t, v.m);
  return u32x4v{(uint32_t)mb, (uint32_t)(mb >> 32), (uint32_t)v.e, 0u};
}
// a plain value x * 2^sc as a record (not normalised: every reader normalises)
__device__ __forceinline__ u32x4v plain_rec(double x, int sc) {
  const uint64_t mb = __builtin_bit_cast(uint64_t, x);
  return u32x4v{(uint32_t)mb, (uint32_t)(mb >> 32), (uint32_t)sc, 0u};
}

// A plain value enters a lane: v = m 2^e in the lane's scale sc.  A lane that holds no
// value yet (`started` = 0) takes the scale that puts v near 1; `started` becomes an
// all-ones mask once the lane holds a value.  Bit operations only: no branch and no lane
// mask logic on the chain.  The exponent v would have is recorded in `rt` (so an input
// that would underflow to zero in the lane's scale is caught too).
__device__ __forceinline__ double enter(double m, int e, int& sc, int& started, RangeTrack& rt) {
  const uint32_t hi = (uint32_t)((uint64_t)__double_as_longlong(m) >> 32);
  const int nz = -(int)min((hi >> 20) & 0x7ffu, 1u);  // all ones for a normal non-zero m
  const int em = __builtin_amdgcn_frexp_exp(m);
  const int keep = started | ~nz;  // keep the scale: the lane holds a value, or m is zero
  sc = (keep & sc) | (~keep & (e + em));
  started |= nz;
  rt.add_exp((e + em - sc) & nz);
  return ldexp(m, e - sc);
}

// Running geometry of one diagonal of the padded box: the position of its first node
// (diag_off), its smallest u and its node count, stepped one diagonal at a time with a
// few selects (the closed forms take 64-bit arithmetic and branches).
struct DiagCursor {
  int k, off, ulo, len;
  __device__ __forceinline__ void init(const Params& p, int k0) {
    k = k0;
    off = (int)diag_off(p, k0);
    ulo = diag_ulo(p, k0);
    len = diag_len(p, k0);
  }
  // sign bit of x as 0 / 1
  static __device__ __forceinline__ int neg(int x) { return (int)((unsigned)x >> 31); }
  __device__ __forceinline__ void next(const Params& p) {  // k -> k + 1
    off += len;
    ++k;
    // the diagonal gains a node at the top while k < U1max, loses one at t = Tmax once k >= Tmax
    const int lo = 1 - neg(k - p.Tmax);
    len += neg(k - p.U1max) - lo;
    ulo += lo;
  }
  __device__ __forceinline__ void prev(const Params& p) {  // k -> k - 1
    const int lo = 1 - neg(k - p.Tmax);
    len -= neg(k - p.U1max) - lo;
    ulo -= lo;
    --k;
    off -= len;
  }
  // first 16-byte entry of the diagonal's plain-weight block
  __device__ __forceinline__ int pw_block(const Params& p) const { return p.NP * (off + 3 * k); }
};

// Buffer resource over `bytes` bytes at `base` (range-checked: out-of-range loads read 0,
// out-of-range stores are dropped).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

// position of node (t, u) relative to its utterance
__device__ __forceinline__ int64_t rel_pos(const Params& p, int t, int u) {
  const int k = t + u;
  return diag_off(p, k) + (u - diag_ulo(p, k));
}

// The NP slot pairs of R labels' plain weights (v[s][r] = weight slot s of label r), the
// boundary records and the position base of one step's diagonal.
template <int DM, int R>
struct WPlain {
  static constexpr int NP = DM + 1;
  double v[2 * NP][R];
  u32x4v x0, x1;  // boundary records: own label's replayed value, and the neighbour's (see callers)
  int dbase;      // position of node (k - u, u) of the diagonal relative to the utterance: dbase + u
};

// Plain weights of the labels u0 + lane R + r (r < R) on the cursor's diagonal, for the
// labels whose node `need`s them (the others read zeros).  Node index i = u - ulo on the
// diagonal; its entry is block + (i % R) ceil(len / R) + i / R: a lane-constant plus a
// uniform part.
template <int DM, int R>
__device__ __forceinline__ void load_weights(const Params& p, __amdgpu_buffer_rsrc_t wr, const DiagCursor& c, int lane,
                                             int u0, const bool (&need)[R], WPlain<DM, R>& w) {
  constexpr int NP = DM + 1;
  const int blk = c.pw_block(p);
  const int cap = c.len + 3;
  const int half = (c.len + R - 1) / R;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int ir = r + u0 - c.ulo;  // i = lane R + ir
    const int col = R == 1 ? lane + ir : (ir & (R - 1)) * half + lane + (ir >> (R == 2 ? 1 : 2));
    const int off = need[r] ? (blk + col) * 16 : kBadOff;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      // the slot pair's offset is uniform: it goes in the scalar offset
      const u32x4v x = __builtin_amdgcn_raw_buffer_load_b128(wr, off, q * cap * 16, 0);
      w.v[2 * q][r] = __builtin_bit_cast(double, ((uint64_t)x.y << 32) | x.x);
      w.v[2 * q + 1][r] = __builtin_bit_cast(double, ((uint64_t)x.w << 32) | x.z);
    }
  }
}

__device__ __forceinline__ double dpp_shift_f64(double x, bool right) {
  const long long bits = __double_as_longlong(x);
  int lo = (int)(bits & 0xffffffffll), hi = (int)(bits >> 32);
  // wave_shr:1 / wave_shl:1; the lane without a source reads 0 (bound_ctrl)
  lo = right ? __builtin_amdgcn_mov_dpp(lo, 0x138, 0xf, 0xf, true) : __builtin_amdgcn_mov_dpp(lo, 0x130, 0xf, 0xf, true);
  hi = right ? __builtin_amdgcn_mov_dpp(hi, 0x138, 0xf, 0xf, true) : __builtin_amdgcn_mov_dpp(hi, 0x130, 0xf, 0xf, true);
  return __longlong_as_double(((long long)(unsigned)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ int dpp_shift_i32(int x, bool right) {
  return right ? __builtin_amdgcn_mov_dpp(x, 0x138, 0xf, 0xf, true) : __builtin_amdgcn_mov_dpp(x, 0x130, 0xf, 0xf, true);
}

// Links between the waves of one work-group that sweep neighbouring label tiles of one
// utterance at the same time: per link an LDS ring of (value, scale) slots indexed by a
// sequence number that grows along the sweep (alpha: the diagonal; beta: T + U minus the
// diagonal), the producer's progress (every slot below it written) and the consumer's
// (every slot below it read).  Waits are bounded: a wait that runs out marks the link
// broken, and the work-group then redoes the utterance with the extended-range sweeps,
// which exchange through memory.
constexpr int kLinkRing = 256;
struct LinkSlot {
  double v;
  int e, pad;
};
struct LinkShared {
  LinkSlot ring[3][kLinkRing];
  int prod[3], cons[3];
  int redo;
};
// the links of a work-group (LDS, used by the linked-tile kernel only)
__shared__ LinkShared g_link;
struct LinkCtx {
  int in, out;    // link read (lane 0 for alpha, lane 63 for beta), link written; -1: none
  int in_last;    // the last sequence number the producer of `in` writes a value for
  int broken;     // a wait ran out
  int spin;       // iterations a wait may take (Params::spin)
};
// Ring slots and progress words are accessed as volatile LDS words: the compiler keeps
// their order, and the LDS performs the accesses of one wave in order, so a consumer that
// reads a progress value sees every slot written before it.  (A memory-model fence would
// also wait for every global load in flight, stalling the weight prefetch.)
#define TDT_LDS __attribute__((address_space(3)))
__device__ __forceinline__ int link_load(const int* c) {
  return __builtin_amdgcn_readfirstlane(*(const TDT_LDS volatile int*)c);
}
__device__ __forceinline__ void link_store(int* c, int v) { *(TDT_LDS volatile int*)c = v; }
// the slot of sequence number sq on link i (volatile: see above)
__device__ __forceinline__ TDT_LDS volatile LinkSlot* link_slot(int i, int sq) {
  return (TDT_LDS volatile LinkSlot*)&g_link.ring[i][sq & (kLinkRing - 1)];
}
// wait until *c >= target (at most lk.spin iterations: about 0.1 s by default)
__device__ __forceinline__ void link_wait(const int* c, int target, LinkCtx& lk) {
  if (lk.broken) return;
  for (int it = 0; it < lk.spin; ++it) {
    if (link_load(c) >= target) return;
    __builtin_amdgcn_s_sleep(2);
  }
  lk.broken = 1;
}

// Plain alpha sweep of a tile.  Returns true when some value left [2^-700, 2^700] (the
// tile is then redone in extended range).
template <int DM, int R, bool BOUND, bool LINK>
__device__ bool alpha_plain(const Params& p, const Tile& tl, int lane, LinkCtx& lk) {
  constexpr int S = ring_size<DM>();
  constexpr int NB = plain_buffers<DM, R>();
  static_assert(NB >= 2 && S % NB == 0, "prefetch buffers must divide the ring");
  static_assert(S >= DM + 2, "ring slots: DM + 1 pending frames and one in flight");
  static_assert(!BOUND || R == 1, "band tiles hold one label per lane");
  static_assert(!LINK || (R == 1 && !BOUND), "linked tiles hold every frame, one label per lane");
  const int b = tl.b;
  const int trl = tl.below ? max(0, tl.t0 - DM) : tl.t0;  // first frame swept (replayed below t0)
  const int kb = trl + tl.u0;
  const int nsteps = tl.t1 - 1 + tl.ulast - kb + 1;
  const int64_t pwe = pw_utt_entries(p.NP, p.box, p.KD);
  const __amdgpu_buffer_rsrc_t wr = rsrc(p.pw + (int64_t)b * pwe * 2, pwe * 16);
  const __amdgpu_buffer_rsrc_t ar = rsrc(p.ar + (int64_t)b * p.box * 16, p.box * 16);
  const int nu64 = (p.U1max + 63) / 64;
  const __amdgpu_buffer_rsrc_t xr = rsrc(p.lx + (int64_t)b * nu64 * p.Tmax * 16, (int64_t)nu64 * p.Tmax * 16);
  const int ub = tl.u0 + lane * R;
  // label r's node at step q is (kb + q - u, u): computed for q in [qa, qa + na), holding
  // weights (computed or replayed) for q in [qn, qn + nn)
  int qa[R], na[R], qn[R], nn[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int u = ub + r;
    const bool in = u <= tl.ulast;
    qa[r] = tl.t0 + u - kb;
    na[r] = in ? tl.t1 - tl.t0 : 0;
    qn[r] = trl + u - kb;
    nn[r] = in ? tl.t1 - trl : 0;
  }
  const int nrep = nn[0] > 0 ? tl.t0 - trl : 0;  // replayed frames of label ub
  double bacc[R][S], lacc[R][S];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int r = 0; r < R; ++r) bacc[r][s] = lacc[r][s] = 0.0;
  int sc = 0, started = 0;
  if (kb == 0 && lane == 0) {  // alpha(0, 0) = 1: the first step's accumulator of label 0
    bacc[0][0] = 1.0;
    started = -1;
  }
  RangeTrack rt;
  double lin = 0.0;  // label contribution into this lane's first label for the coming step
  double lv[LINK ? S : 1], ov[LINK ? S : 1];  // a block's link inputs and outputs
  int le[LINK ? S : 1], oe[LINK ? S : 1];
  WPlain<DM, R> wb[NB];
  DiagCursor cl;  // the diagonal being loaded, NB - 1 steps ahead
  cl.init(p, kb);
  int ql = 0;
  const int xoff = ((ub / 64) * p.Tmax - ub) * 16;  // lx record of frame t = k - ub: xoff + 16 k
  auto load = [&](WPlain<DM, R>& w) {
    bool need[R];
#pragma unroll
    for (int r = 0; r < R; ++r) need[r] = (unsigned)(ql - qn[r]) < (unsigned)nn[r];
    load_weights<DM, R>(p, wr, cl, lane, tl.u0, need, w);
    w.dbase = cl.off - cl.ulo;
    if (BOUND) {
      // x0: the replayed alpha of a frame below the tile; x1 (lane 0): the label moves
      // entering the tile's first label from the left tile
      const bool rep = (unsigned)(ql - qn[0]) < (unsigned)nrep;
      const bool edge = lane == 0 && tl.left && (unsigned)(ql - qa[0]) < (unsigned)na[0];
      w.x0 = __builtin_amdgcn_raw_buffer_load_b128(ar, rep ? (w.dbase + ub) * 16 : kBadOff, 0, 0);
      w.x1 = __builtin_amdgcn_raw_buffer_load_b128(xr, edge ? xoff + 16 * cl.k : kBadOff, 0, 0);
    }
    cl.next(p);
    ++ql;
  };
#pragma unroll
  for (int j = 0; j < NB - 1; ++j) load(wb[j]);
  for (int q0 = 0; q0 < nsteps; q0 += S) {
#pragma unroll
    for (int ph = 0; ph < S; ++ph) {  // steps past the last diagonal touch no node
      const int q = q0 + ph;
      if (LINK && ph == 0 && lk.in >= 0) {
        // this block's inputs (slots up to kb + q0 + S - 2) written: read them all at once
        link_wait(&g_link.prod[lk.in], min(kb + q0 + S - 1, lk.in_last + 1), lk);
#pragma unroll
        for (int j = 0; j < S; ++j) {
          TDT_LDS volatile LinkSlot* sl = link_slot(lk.in, kb + q0 + j - 1);
          lv[j] = sl->v;
          le[j] = sl->e;
        }
      }
      if (ph == 0) {  // keep the lane's pending values near 1 (a zero lane shifts by 0)
        const double big = fmax(fmax(fabs(lin), fabs(bacc[0][0])), fmax(fabs(bacc[0][1]), fabs(lacc[R - 1][0])));
        const int ex = __builtin_amdgcn_frexp_exp(big);
        sc += ex;
        lin = ldexp(lin, -ex);
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
          for (int r = 0; r < R; ++r) {
            bacc[r][s] = ldexp(bacc[r][s], -ex);
            lacc[r][s] = ldexp(lacc[r][s], -ex);
          }
      }
      load(wb[(ph + NB - 1) % NB]);
      const WPlain<DM, R>& w = wb[ph % NB];
      if (BOUND) {  // lane 0: the first label's input from the left tile (zero when not loaded)
        const Ext x = rec_ext(w.x1);
        const double e1 = enter(x.m, x.e, sc, started, rt);
        lin = (lane == 0 && tl.left) ? e1 : lin;
      }
      if (LINK && lk.in >= 0) {  // lane 0: the left wave's label move of diagonal kb + q - 1
        const double e1 = enter((lane == 0 && kb + q - 1 <= lk.in_last) ? lv[ph] : 0.0, le[ph], sc, started, rt);
        lin = lane == 0 ? e1 : lin;
      }
      double a[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const bool act = (unsigned)(q - qa[r]) < (unsigned)na[r];
        const double in = r == 0 ? lin : lacc[r > 0 ? r - 1 : 0][(ph + S - 1) % S];
        double v = act ? bacc[r][ph] + in : 0.0;
        if (BOUND && r == 0) {  // a replayed frame below the tile (zero when not loaded)
          const Ext x = rec_ext(w.x0);
          const double vr = enter(x.m, x.e, sc, started, rt);
          v = (unsigned)(q - qn[0]) < (unsigned)nrep ? vr : v;
        }
        rt.add(v);
        a[r] = v;
        __builtin_amdgcn_raw_buffer_store_b128(plain_rec(v, sc), ar, act ? (w.dbase + ub + r) * 16 : kBadOff, 0, 0);
      }
      // push the new values along their outgoing moves; the first contribution to a
      // ring slot (duration DM) replaces its consumed value
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int d = 1; d < DM; ++d) bacc[r][(ph + d) % S] = fma(a[r], w.v[d - 1][r], bacc[r][(ph + d) % S]);
        bacc[r][(ph + DM) % S] = a[r] * w.v[DM - 1][r];
#pragma unroll
        for (int d = 0; d < DM; ++d) lacc[r][(ph + d) % S] = fma(a[r], w.v[DM + d][r], lacc[r][(ph + d) % S]);
        lacc[r][(ph + DM) % S] = a[r] * w.v[2 * DM][r];
      }
      // the complete label contribution into (t, u + 1) of the last label goes to the next lane
      const double out = lacc[R - 1][ph];
      if (BOUND) {  // ... or, from lane 63, to the tile on the right
        // record of column ub / 64 + 1 (lane 63: ub % 64 == 63) at frame t = k - ub
        const bool edge = lane == 63 && tl.right && (unsigned)(q - qa[0]) < (unsigned)na[0];
        __builtin_amdgcn_raw_buffer_store_b128(plain_rec(out, sc), xr, edge ? xoff + p.Tmax * 16 + 16 * (kb + q) : kBadOff,
                                               0, 0);
      }
      if (LINK) {  // for the right wave (lane 63's values, written at the block's end)
        ov[ph] = out;
        oe[ph] = sc;
      }
      lin = enter(dpp_shift_f64(out, true), dpp_shift_i32(sc, true), sc, started, rt);
    }
    if (LINK) {
      if (lk.out >= 0) {
        link_wait(&g_link.cons[lk.out], kb + q0 + S - kLinkRing, lk);  // the slots are free
        if (lane == 63) {
#pragma unroll
          for (int j = 0; j < S; ++j) {
            TDT_LDS volatile LinkSlot* sl = link_slot(lk.out, kb + q0 + j);
            sl->v = ov[j];
            sl->e = oe[j];
          }
        }
        link_store(&g_link.prod[lk.out], kb + q0 + S);
      }
      if (lk.in >= 0) link_store(&g_link.cons[lk.in], kb + q0 + S - 1);
    }
  }
  return rt.bad();
}

// Plain beta sweep of a tile (pull form).  *P00 receives beta(0, 0) when the tile holds
// node (0, 0) (lane 0).  Returns true when some value left [2^-700, 2^700].
template <int DM, int R, bool BOUND, bool LINK>
__device__ bool beta_plain(const Params& p, const Tile& tl, int lane, Ext* P00, LinkCtx& lk) {
  constexpr int S = ring_size<DM>();
  constexpr int NB = plain_buffers<DM, R>();
  static_assert(NB >= 2 && S % NB == 0, "prefetch buffers must divide the ring");
  const int b = tl.b, T = tl.T, U = tl.U;
  const int rtop = min(tl.t1 + DM - 1, T);  // highest frame swept (replayed above t1, or the terminal)
  // the sweep starts one diagonal higher when a tile lies to the right and frames above:
  // the label move of duration DM out of the top-right node lands on that diagonal
  const int kb = rtop + tl.ulast + (tl.right && rtop < T ? 1 : 0);
  const int nsteps = kb - (tl.t0 + tl.u0) + 1;
  const int64_t pwe = pw_utt_entries(p.NP, p.box, p.KD);
  const __amdgpu_buffer_rsrc_t wr = rsrc(p.pw + (int64_t)b * pwe * 2, pwe * 16);
  const __amdgpu_buffer_rsrc_t br = rsrc(p.br + (int64_t)b * p.box * 16, p.box * 16);
  const int ub = tl.u0 + lane * R;
  const int un = tl.u0 + 64 * R;  // the label right of the tile (read by lane 63)
  // label r's node at step q is (kb - q - u, u): computed for q in [qa, qa + na)
  int qa[R], na[R];
  bool term[R];  // the terminal (T, U): beta = 1 at step 0 (its diagonal is the first)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int u = ub + r;
    const bool in = u <= tl.ulast;
    qa[r] = kb - u - tl.t1 + 1;
    na[r] = in ? tl.t1 - tl.t0 : 0;
    term[r] = u == U && rtop == T;
  }
  // replayed frames above the tile of label ub: t in [t1, rr], at steps [qr, qr + nr)
  const int rr = min(tl.t1 + DM - 1, T - 1);
  const int qr = kb - ub - rr;
  const int nr = (tl.above && ub <= tl.ulast) ? rr - tl.t1 + 1 : 0;
  double h[R][S], nb[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    nb[s] = 0.0;
#pragma unroll
    for (int r = 0; r < R; ++r) h[r][s] = 0.0;
  }
  int sc = 0, started = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) started = term[r] ? -1 : started;  // the terminal starts its lane at scale 0
  RangeTrack rt;
  double lv[LINK ? S : 1], ov[LINK ? S : 1];  // a block's link inputs and outputs
  int le[LINK ? S : 1], oe[LINK ? S : 1];
  WPlain<DM, R> wb[NB];
  // the diagonal being loaded, NB - 1 steps ahead (kb may be one past the box's last
  // diagonal: the terminal of an utterance as long as the box; the closed forms hold there)
  DiagCursor cl;
  cl.init(p, kb);
  int ql = 0;
  auto load = [&](WPlain<DM, R>& w) {
    bool need[R];
#pragma unroll
    for (int r = 0; r < R; ++r) need[r] = (unsigned)(ql - qa[r]) < (unsigned)na[r];
    load_weights<DM, R>(p, wr, cl, lane, tl.u0, need, w);
    w.dbase = cl.off - cl.ulo;
    if (BOUND) {
      // x0: the replayed beta of a frame above the tile; x1 (lane 63): the beta of the
      // label right of the tile on this diagonal
      const int tn = cl.k - un;
      const bool rep = (unsigned)(ql - qr) < (unsigned)nr;
      const bool edge = lane == 63 && tl.right && tn >= tl.t0 && tn < T;
      w.x0 = __builtin_amdgcn_raw_buffer_load_b128(br, rep ? (w.dbase + ub) * 16 : kBadOff, 0, 0);
      w.x1 = __builtin_amdgcn_raw_buffer_load_b128(br, edge ? (w.dbase + un) * 16 : kBadOff, 0, 0);
    }
    cl.prev(p);
    ++ql;
  };
#pragma unroll
  for (int j = 0; j < NB - 1; ++j) load(wb[j]);
  for (int q0 = 0; q0 < nsteps; q0 += S) {
#pragma unroll
    for (int ph = 0; ph < S; ++ph) {  // steps past the last diagonal touch no node
      const int q = q0 + ph;
      const int sq = T + U - (kb - q);  // link sequence number of this step's diagonal kb - q
      if (LINK && ph == 0 && lk.in >= 0) {  // this block's inputs written: read them at once
        link_wait(&g_link.prod[lk.in], min(sq + S, lk.in_last + 1), lk);
#pragma unroll
        for (int j = 0; j < S; ++j) {
          TDT_LDS volatile LinkSlot* sl = link_slot(lk.in, sq + j);
          lv[j] = sl->v;
          le[j] = sl->e;
        }
      }
      if (ph == 0) {  // keep the lane's newest values near 1
        const double big = fmax(fabs(h[0][S - 1]), fabs(nb[S - 1]));
        const int ex = __builtin_amdgcn_frexp_exp(big);
        sc += ex;
#pragma unroll
        for (int s = 0; s < S; ++s) {
          nb[s] = ldexp(nb[s], -ex);
#pragma unroll
          for (int r = 0; r < R; ++r) h[r][s] = ldexp(h[r][s], -ex);
        }
      }
      load(wb[(ph + NB - 1) % NB]);
      const WPlain<DM, R>& w = wb[ph % NB];
      double a[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const bool act = (unsigned)(q - qa[r]) < (unsigned)na[r];
        double c0 = 0.0, c1 = 0.0, c2 = 0.0, c3 = 0.0;
#pragma unroll
        for (int d = 1; d <= DM; ++d) {
          const double x = w.v[d - 1][r] * h[r][(ph - d + 4 * S) % S];
          if (d & 1) c0 += x;
          else c1 += x;
        }
#pragma unroll
        for (int d = 0; d <= DM; ++d) {
          const int sl = (ph - 1 - d + 4 * S) % S;
          const double dst = r < R - 1 ? h[r < R - 1 ? r + 1 : 0][sl] : nb[sl];
          const double x = w.v[DM + d][r] * dst;
          if (d & 1) c3 += x;
          else c2 += x;
        }
        double v = act ? (c0 + c1) + (c2 + c3) : 0.0;
        v = (term[r] && q == 0) ? ldexp(1.0, -sc) : v;
        if (BOUND && r == 0) {  // a replayed frame above the tile (zero when not loaded)
          const Ext x = rec_ext(w.x0);
          const double vr = enter(x.m, x.e, sc, started, rt);
          v = (unsigned)(q - qr) < (unsigned)nr ? vr : v;
        }
        rt.add(v);
        a[r] = v;
        __builtin_amdgcn_raw_buffer_store_b128(plain_rec(v, sc), br, act ? (w.dbase + ub + r) * 16 : kBadOff, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) h[r][ph] = a[r];
      // the beta of the label after this lane's last one, on this diagonal: the next
      // lane's first label (DPP wave shift), or the tile on the right for lane 63
      double m = dpp_shift_f64(a[0], false);
      int e = dpp_shift_i32(sc, false);
      if (BOUND) {
        const Ext x = rec_ext(w.x1);
        m = lane == 63 ? x.m : m;
        e = lane == 63 ? x.e : e;
      }
      if (LINK && lk.in >= 0) {  // lane 63: the right wave's first label on this diagonal
        const int tn = kb - q - un;
        m = lane == 63 ? ((tn >= 0 && tn < T) ? lv[ph] : 0.0) : m;
        e = lane == 63 ? le[ph] : e;
      }
      if (LINK) {  // for the left wave (lane 0's values, written at the block's end)
        ov[ph] = a[0];
        oe[ph] = sc;
      }
      nb[ph] = enter(m, e, sc, started, rt);
    }
    if (LINK) {
      const int sq0 = T + U - (kb - q0);
      if (lk.out >= 0) {
        link_wait(&g_link.cons[lk.out], sq0 + S - kLinkRing, lk);  // the slots are free
        if (lane == 0) {
#pragma unroll
          for (int j = 0; j < S; ++j) {
            TDT_LDS volatile LinkSlot* sl = link_slot(lk.out, sq0 + j);
            sl->v = ov[j];
            sl->e = oe[j];
          }
        }
        link_store(&g_link.prod[lk.out], sq0 + S);
      }
      if (lk.in >= 0) link_store(&g_link.cons[lk.in], sq0 + S);
    }
  }
  if (lane == 0 && tl.t0 == 0 && tl.u0 == 0) {  // beta(0, 0): the last step's value of lane 0
    const int last = (nsteps - 1) % S;
    double b00 = h[0][0];
#pragma unroll
    for (int s = 1; s < S; ++s) b00 = s == last ? h[0][s] : b00;
    int ex;
    const double mm = frexp(b00, &ex);
    *P00 = b00 != 0.0 ? Ext{mm, ex + sc} : ext_zero();
  }
  return rt.bad();
}

// ---- extended-range sweeps (one label per lane, no prefetch; the rare path) ----

__device__ __forceinline__ Ext ext_add(Ext a, Ext b) {
  const int E = max(a.e, b.e);
  return ext_norm(ldexp(a.m, a.e - E) + ldexp(b.m, b.e - E), E);
}

// The 2 DM + 1 outgoing weights of node (t, u) in extended range, from its log-domain
// ingredients (zero for absent durations and moves that leave the lattice).
template <int DM>
__device__ __forceinline__ void ext_weights(const Params& p, int b, int t, int u, int T, int U, Ext (&w)[2 * DM + 1]) {
  const double* lg = p.lg + ((int64_t)b * p.box + rel_pos(p, t, u)) * p.LG;
  const double lb = lg[0], ly = lg[1];
#pragma unroll
  for (int d = 0; d <= DM; ++d) {
    const int idx = p.didx[d];
    const double lam = idx >= 0 ? lg[2 + idx] : -__builtin_inf();
    if (d >= 1) w[d - 1] = (t + d < T || (t + d == T && u == U)) ? ext_exp(lb + lam) : ext_zero();
    w[DM + d] = (u < U && t + d < T) ? ext_exp(ly + lam) : ext_zero();
  }
}

__device__ __forceinline__ Ext dpp_shift_ext(Ext v, bool right) {
  const long long bits = __double_as_longlong(v.m);
  int lo = (int)(bits & 0xffffffffll), hi = (int)(bits >> 32), e = v.e;
  if (right) {  // lane i receives lane i - 1 (wave_shr:1); lane 0 receives the zero
    lo = __builtin_amdgcn_update_dpp(0, lo, 0x138, 0xf, 0xf, false);
    hi = __builtin_amdgcn_update_dpp(0, hi, 0x138, 0xf, 0xf, false);
    e = __builtin_amdgcn_update_dpp(kEZ, e, 0x138, 0xf, 0xf, false);
  } else {  // lane i receives lane i + 1 (wave_shl:1); lane 63 receives the zero
    lo = __builtin_amdgcn_update_dpp(0, lo, 0x130, 0xf, 0xf, false);
    hi = __builtin_amdgcn_update_dpp(0, hi, 0x130, 0xf, 0xf, false);
    e = __builtin_amdgcn_update_dpp(kEZ, e, 0x130, 0xf, 0xf, false);
  }
  return Ext{__longlong_as_double(((long long)(unsigned)hi << 32) | (unsigned)lo), e};
}

// Loads of records written earlier by this same wave go around the vector L1 (sc0).
__device__ __forceinline__ Ext load_ext_rec(__amdgpu_buffer_rsrc_t r, int off) {
  return rec_ext(__builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 1));
}

// Extended-range alpha sweep of a tile of at most 64 labels (push form, as alpha_plain).
// The accumulators are kept aligned to the current step (index d: the frame d steps
// ahead) and shifted after each step, so the loop needs no unrolling.
template <int DM>
__device__ void alpha_ext(const Params& p, const Tile& tl, int lane) {
  constexpr int NW = 2 * DM + 1;
  const int b = tl.b, T = tl.T, U = tl.U;
  const int trl = tl.below ? max(0, tl.t0 - DM) : tl.t0;
  const int kb = trl + tl.u0;
  const int nsteps = tl.t1 - 1 + tl.ulast - kb + 1;
  const __amdgpu_buffer_rsrc_t ar = rsrc(p.ar + (int64_t)b * p.box * 16, p.box * 16);
  const int nu64 = (p.U1max + 63) / 64;
  const __amdgpu_buffer_rsrc_t xr = rsrc(p.lx + (int64_t)b * nu64 * p.Tmax * 16, (int64_t)nu64 * p.Tmax * 16);
  const int u = tl.u0 + lane;
  Ext bacc[DM + 1], lacc[DM + 1];  // contributions to (t + d, u) and to (t + d, u + 1)
#pragma unroll
  for (int d = 0; d <= DM; ++d) bacc[d] = lacc[d] = ext_zero();
  Ext lin = ext_zero();
  for (int q = 0; q < nsteps; ++q) {
    const int k = kb + q, t = k - u;
    const bool inl = u <= tl.ulast;
    const bool act = inl && t >= tl.t0 && t < tl.t1;
    const bool rep = inl && t >= trl && t < tl.t0;
    if (lane == 0 && tl.left) lin = act ? load_ext_rec(xr, ((u / 64) * p.Tmax + t) * 16) : ext_zero();
    Ext v = ext_zero();
    if (act) v = k == 0 ? ext_one() : ext_add(bacc[0], lin);
    if (rep) v = load_ext_rec(ar, (int)(rel_pos(p, t, u) * 16));
    if (act) __builtin_amdgcn_raw_buffer_store_b128(ext_rec(v), ar, (int)(rel_pos(p, t, u) * 16), 0, 0);
    Ext w[NW];
    if (act || rep) {
      ext_weights<DM>(p, b, t, u, T, U, w);
    } else {
#pragma unroll
      for (int s2 = 0; s2 < NW; ++s2) w[s2] = ext_zero();
    }
#pragma unroll
    for (int d = 1; d <= DM; ++d) bacc[d] = ext_add(bacc[d], ext_mul(v, w[d - 1]));
#pragma unroll
    for (int d = 0; d <= DM; ++d) lacc[d] = ext_add(lacc[d], ext_mul(v, w[DM + d]));
    const Ext out = lacc[0];
#pragma unroll
    for (int d = 0; d < DM; ++d) {
      bacc[d] = bacc[d + 1];
      lacc[d] = lacc[d + 1];
    }
    bacc[DM] = lacc[DM] = ext_zero();
    if (lane == 63 && tl.right && t >= tl.t0 && t < tl.t1)
      __builtin_amdgcn_raw_buffer_store_b128(ext_rec(out), xr, (((u + 1) / 64) * p.Tmax + t) * 16, 0, 0);
    lin = dpp_shift_ext(out, true);
  }
}

// Extended-range beta sweep of a tile of at most 64 labels (pull form; the histories of
// the own label and of the next one are kept aligned to the current step: index d holds
// the frame d steps ahead).
template <int DM>
__device__ void beta_ext(const Params& p, const Tile& tl, int lane, Ext* P00) {
  constexpr int NW = 2 * DM + 1;
  const int b = tl.b, T = tl.T, U = tl.U;
  const int rtop = min(tl.t1 + DM - 1, T);
  const int kb = rtop + tl.ulast + (tl.right && rtop < T ? 1 : 0);  // as in beta_plain
  const int nsteps = kb - (tl.t0 + tl.u0) + 1;
  const __amdgpu_buffer_rsrc_t br = rsrc(p.br + (int64_t)b * p.box * 16, p.box * 16);
  const int u = tl.u0 + lane, un = tl.u0 + 64;
  Ext h[DM + 1], nb[DM + 2];  // h[d] = beta(t + d, u), nb[d] = beta(t - 1 + d, u + 1)
#pragma unroll
  for (int d = 0; d <= DM; ++d) h[d] = ext_zero();
#pragma unroll
  for (int d = 0; d <= DM + 1; ++d) nb[d] = ext_zero();
  Ext b00 = ext_zero();
  for (int q = 0; q < nsteps; ++q) {
    const int k = kb - q, t = k - u;
    const bool inl = u <= tl.ulast;
    const bool act = inl && t >= tl.t0 && t < tl.t1;
    Ext v = ext_zero();
    if (act) {
      Ext w[NW];
      ext_weights<DM>(p, b, t, u, T, U, w);
      Ext terms[NW];
#pragma unroll
      for (int d = 1; d <= DM; ++d) terms[d - 1] = ext_mul(w[d - 1], h[d]);
#pragma unroll
      for (int d = 0; d <= DM; ++d) terms[DM + d] = ext_mul(w[DM + d], nb[d + 1]);
      v = ext_sum(terms);
      __builtin_amdgcn_raw_buffer_store_b128(ext_rec(v), br, (int)(rel_pos(p, t, u) * 16), 0, 0);
      if (k == 0) b00 = v;
    } else if (t == T && u == U) {
      v = ext_one();
    } else if (inl && tl.above && t >= tl.t1 && t < T) {
      v = load_ext_rec(br, (int)(rel_pos(p, t, u) * 16));
    }
    // the next label's value on this diagonal: beta(t - 1, u + 1)
    Ext n = dpp_shift_ext(v, false);
    if (lane == 63) {
      const int tn = k - un;
      n = ext_zero();
      if (tn == T && un == U) n = ext_one();
      if (tl.right && tn >= tl.t0 && tn < T) n = load_ext_rec(br, (int)(rel_pos(p, tn, un) * 16));
    }
    // step to the diagonal below: frame t - 1 of this label
#pragma unroll
    for (int d = DM; d >= 1; --d) h[d] = h[d - 1];
    h[1] = v;
#pragma unroll
    for (int d = DM + 1; d >= 1; --d) nb[d] = nb[d - 1];
    nb[1] = n;
  }
  if (lane == 0 && tl.t0 == 0 && tl.u0 == 0) *P00 = b00;
}

// Status, reduction weight, log P and the gradient flag of utterance b, by the tile that
// holds node (0, 0) in the beta direction (after its sweep, P = beta(0, 0)).
__device__ void finish_utterance(const Params& p, int b, Ext P, int lane) {
  const int64_t T64 = p.Tlen[b], U64 = p.Ulen[b];
  int status = 0;
  if (T64 < 0 || T64 > p.Tmax) status |= 1;
  if (U64 < 0 || U64 > p.U1max - 1) status |= 2;
  bool bad = false;
  if (!(status & 2))
    for (int64_t u = lane; u < U64; u += 64) {
      const int64_t y = p.labels[(int64_t)b * p.lab_stride + u];
      bad |= (y < 0 || y >= p.V);
    }
  if (__any(bad)) status |= 4;
  int64_t sumU = 0;
  if (p.red == 4) {
    for (int bb = lane; bb < p.B; bb += 64) sumU += p.Ulen[bb];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sumU += __shfl_xor(sumU, o, 64);
  }
  if (lane != 0) return;
  p.wts[b] = reduction_weight(p, b, sumU);
  if (status != 0 || T64 == 0) {
    p.logp[b] = status ? __builtin_nan("") : -__builtin_inf();
    p.pm[b] = 0.0;
    p.pe[b] = kEZ;
    p.uok[b] = 0;
    if (p.ustatus) p.ustatus[b] = status ? status : 8;
    return;
  }
  const double lp = ext_log(P);
  p.logp[b] = lp;
  p.pm[b] = P.m;
  p.pe[b] = P.e;
  p.uok[b] = (P.m > 0.0 && lp == lp) ? 1 : 0;
  if (p.ustatus) p.ustatus[b] = (P.m > 0.0 || lp != lp) ? 0 : 8;
}

// Zero bytes [x, y) of a range shorter than 128 bytes (x, y multiples of the element size
// elt) by 24 lanes, l = 0 .. 23: whole 16-byte chunks by l < 8, the elements before the
// first chunk by l = 8 .. 15 and those after the last one by l = 16 .. 23.
__device__ __forceinline__ void zero_short(char* x, char* y, int elt, int l) {
  char* x16 = (char*)(((uintptr_t)x + 15) & ~(uintptr_t)15);
  char* y16 = (char*)((uintptr_t)y & ~(uintptr_t)15);
  char* c = l < 8 ? x16 + 16 * l : (l < 16 ? x + (l - 8) * elt : (x16 > y16 ? x16 : y16) + (l - 16) * elt);
  if (l < 8) {
    if (c < y16) __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, (TDT_GLOBAL u32x4*)c);
  } else if (c < (l < 16 ? (x16 < y ? x16 : y) : y)) {
    if (elt == 4) *(TDT_GLOBAL uint32_t*)c = 0u;
    else *(TDT_GLOBAL uint16_t*)c = (uint16_t)0;
  }
}

// Zero the gradient rows of the padded box that lie outside their utterance's lattice
// (t >= T, u > U, or lengths out of range), for a gradient laid out as one contiguous
// joint tensor [B, Tmax, U1max, V + D] (the host checks the strides): the padding rows of
// frame (b, t) are then one contiguous byte range.  Its whole 128-byte lines are zeroed
// with 16-byte nontemporal stores, eight lines per wave store (a partly written line costs
// the memory a read-modify-write), its two ends of under 128 bytes piece by piece.  Wave w
// of nw takes the frames w, w + nw, ...
__device__ void zero_padded_rows(const Params& p, uint32_t w, uint32_t nw, int lane) {
  const uint32_t frames = (uint32_t)p.B * (uint32_t)p.Tmax;
  const int elt = p.dtype == 0 ? 4 : 2;
  const int64_t rowb = (int64_t)p.gs2 * elt;  // bytes of one joint row (V + D elements)
  for (uint32_t f = w; f < frames; f += nw) {
    const uint32_t b = f / (uint32_t)p.Tmax;
    const int t = (int)(f - b * (uint32_t)p.Tmax);
    const int64_t T64 = p.Tlen[b], U64 = p.Ulen[b];
    const int ulo = (utt_dims_ok(p, T64, U64) && t < (int)T64) ? (int)U64 + 1 : 0;  // first padding row
    if (ulo >= p.U1max) continue;
    char* lo = (char*)p.gtok + ((int64_t)b * p.gs0 + (int64_t)t * p.gs1 + (int64_t)ulo * p.gs2) * elt;
    char* hi = lo + (p.U1max - ulo) * rowb;
    char* a = (char*)(((uintptr_t)lo + 127) & ~(uintptr_t)127);
    char* e = (char*)((uintptr_t)hi & ~(uintptr_t)127);
    if (a > e) a = e = hi;  // inside one line: the head is the whole range
    for (char* c = a + 16 * lane; c < e; c += 16 * 64)
      __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, (TDT_GLOBAL u32x4*)c);
    if (lane < 24) zero_short(lo, a, elt, lane);
    else if (lane < 48) zero_short(e, hi, elt, lane - 24);
  }
}

// Tiles of band `band` (i + j = band for alpha, counted from the far corner for beta):
// one 64-lane work-group per (tile, utterance, direction).  R labels per lane (R = 2 only
// for a single tile); BOUND: tiles with neighbours (band tiles of 64 labels).  The plain
// sweep runs unless the utterance has move weights outside [2^-300, 2^300] or the plain
// weights are not stored; a tile whose plain sweep went out of range is redone in
// extended range, one 64-label strip after another.
template <int DM, int R, bool BOUND>
__global__ __launch_bounds__(64) void k_tiles(const Params p, int band) {
  const int lane = threadIdx.x;
  const int ilo = max(0, band - (p.nU - 1)), ihi = min(band, p.nT - 1);
  const int ntile = ihi - ilo + 1;
  const uint32_t tile_blocks = (uint32_t)ntile * 2u * (uint32_t)p.B;
  if (blockIdx.x >= tile_blocks) {  // the first band's launch also zeroes the padding rows
    zero_padded_rows(p, blockIdx.x - tile_blocks, gridDim.x - tile_blocks, lane);
    return;
  }
  const int m = blockIdx.x % ntile, rest = blockIdx.x / ntile;
  const int dir = rest & 1, b = rest >> 1;
  int i = ilo + m, j = band - i;
  if (dir == 1) {
    i = p.nT - 1 - i;
    j = p.nU - 1 - j;
  }
  const int64_t T64 = p.Tlen[b], U64 = p.Ulen[b];
  Ext P = ext_zero();
  if (utt_dims_ok(p, T64, U64)) {
    const int T = (int)T64, U = (int)U64;
    Tile tl;
    if (make_tile(p, b, T, U, i, j, 64 * R, tl)) {
      bool redo = true;
      if constexpr (plain_buffers<DM, R>() >= 2) {
        LinkCtx none{-1, -1, 0, 0, p.spin};
        if (p.pw && !p.xflag[b]) redo = dir == 0 ? alpha_plain<DM, R, BOUND, false>(p, tl, lane, none)
                                                 : beta_plain<DM, R, BOUND, false>(p, tl, lane, &P, none);
      }
      // the sweeps run as one wavefront across the lanes: the whole wave redoes the tile
      // when any lane saw a value out of range
      if (__any(redo)) {
        // extended range, 64-label strips in dependency order (the strips of one tile
        // exchange through lx / br within this wave: stores complete before the next
        // strip's loads, which bypass the vector L1)
        for (int s = 0; s < R; ++s) {
          const int sj = dir == 0 ? s : R - 1 - s;
          Tile st = tl;
          st.u0 = tl.u0 + 64 * sj;
          if (st.u0 > U) continue;
          st.ulast = min(st.u0 + 63, U);
          st.left = st.u0 > 0;
          st.right = st.ulast < U;
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
          if (dir == 0) alpha_ext<DM>(p, st, lane);
          else beta_ext<DM>(p, st, lane, &P);
        }
      }
    }
  }
  if (dir == 1 && i == 0 && j == 0) finish_utterance(p, b, P, lane);
}

// Linked tiles: one work-group of nU <= 4 waves per (utterance, direction), wave w sweeping
// labels 64 w .. 64 w + 63 over every frame; for alpha wave w takes the label moves into
// its first label from wave w - 1, for beta its last lane takes the beta of label 64 w + 64
// from wave w + 1, both through the LDS links, so the waves run at once, each behind its
// producer by about 64 diagonals, and the utterance takes about T + U steps.  A wave whose
// plain sweep went out of range (or a link wait that ran out) makes wave 0 redo the whole
// utterance in extended range, strip after strip.  Extra work-groups zero the gradient's
// padding rows (as in k_tiles).
template <int DM>
__global__ __launch_bounds__(256) void k_tiles_link(const Params p) {
  LinkShared& sh = g_link;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int W = (int)(blockDim.x >> 6);
  const uint32_t tile_blocks = 2u * (uint32_t)p.B;
  if (blockIdx.x >= tile_blocks) {
    zero_padded_rows(p, (blockIdx.x - tile_blocks) * W + w, (gridDim.x - tile_blocks) * W, lane);
    return;
  }
  const int dir = blockIdx.x & 1, b = blockIdx.x >> 1;
  const int64_t T64 = p.Tlen[b], U64 = p.Ulen[b];
  const bool dims = utt_dims_ok(p, T64, U64);
  const int T = dims ? (int)T64 : 0, U = dims ? (int)U64 : 0;
  const int nw = dims ? min(W, U / 64 + 1) : 0;  // waves holding labels
  if (threadIdx.x == 0) {
    sh.redo = 0;
    for (int i = 0; i < 3; ++i) {
      // nothing written yet; every slot before the consumer's first one consumed
      sh.prod[i] = -(1 << 30);
      sh.cons[i] = dir == 0 ? 64 * (i + 1) - 1 : U - min(64 * i + 63, U);
    }
  }
  __syncthreads();
  Ext P = ext_zero();
  Tile tl;
  const bool have = w < nw && make_tile(p, b, T, U, 0, w, 64, tl);
  bool redo = false;
  if (have) {
    redo = true;
    if constexpr (plain_buffers<DM, 1>() >= 2) {
      if (p.pw && !p.xflag[b]) {
        LinkCtx lk{-1, -1, 0, 0, p.spin};
        if (dir == 0) {
          lk.in = w > 0 ? w - 1 : -1;
          lk.out = w + 1 < nw ? w : -1;
          lk.in_last = T + tl.u0 - 2;
          redo = alpha_plain<DM, 1, false, true>(p, tl, lane, lk);
        } else {
          lk.in = w + 1 < nw ? w : -1;
          lk.out = w > 0 ? w - 1 : -1;
          lk.in_last = T + U - (tl.u0 + 64);
          redo = beta_plain<DM, 1, false, true>(p, tl, lane, &P, lk);
        }
        redo = redo || lk.broken;
      }
    }
  }
  if (__any(redo) && lane == 0) __hip_atomic_store(&sh.redo, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __syncthreads();
  if (sh.redo && w == 0 && nw > 0) {
    // extended range, 64-label strips in dependency order (the strips exchange through lx
    // / br within this wave: stores complete before the next strip's loads, which bypass
    // the vector L1)
    for (int s = 0; s < nw; ++s) {
      const int sj = dir == 0 ? s : nw - 1 - s;
      Tile st;
      if (!make_tile(p, b, T, U, 0, sj, 64, st)) continue;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (dir == 0) alpha_ext<DM>(p, st, lane);
      else beta_ext<DM>(p, st, lane, &P);
    }
  }
  if (dir == 1 && w == 0) finish_utterance(p, b, P, lane);
}

// ---- label columns linked across work-groups ----
// Device-scope loads and stores: on this GPU they bypass the L2 of the XCD that issues
// them, so work-groups on different XCDs see each other's values.
__device__ __forceinline__ int xload_i32(const int* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void xstore_i32(int* a, int v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double xload_f64(const double* a) {
  return __longlong_as_double(
      (long long)__hip_atomic_load((const unsigned long long*)a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void xstore_f64(double* a, double v) {
  __hip_atomic_store((unsigned long long*)a, (unsigned long long)__double_as_longlong(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 1 of a column work-group: carries the column's LDS links to and from its
// neighbours' work-groups.  In: slots the neighbour published (ring in global memory,
// progress word) are copied into LDS ring 0 once the sweep has freed their places, then
// LDS progress 0 is raised.  Out: slots the sweep wrote into LDS ring 1 are copied to
// the global ring, and once every one of those stores has completed (s_waitcnt) the
// progress word is raised, then LDS ring 1's places are freed.  The global rings hold
// every sequence number of a link, so they need no flow control.  Returns false when no
// slot moved for p.spin polls (about 0.1 s by default: a neighbour that did not run).
__device__ bool column_bridge(const Params& p, int b, int dir, int j, int ncol, int T, int U, int lane) {
  const int in_link = dir == 0 ? (j > 0 ? j - 1 : -1) : (j + 1 < ncol ? j : -1);
  const int out_link = dir == 0 ? (j + 1 < ncol ? j : -1) : (j > 0 ? j - 1 : -1);
  const int bd = b * 2 + dir;
  // the first sequence number the consumer of link i reads, and the last
  auto first = [&](int i) { return dir == 0 ? 64 * (i + 1) - 1 : U - min(64 * i + 63, U); };
  auto last = [&](int i) { return dir == 0 ? T + 64 * (i + 1) - 2 : T + U - (64 * i + 64); };
  int in_next = 0, in_end = 0, out_next = 0, out_end = 0;
  const int* gin = nullptr;
  int* gout = nullptr;
  const char* rin = nullptr;
  char* rout = nullptr;
  if (in_link >= 0) {
    in_next = first(in_link);
    in_end = last(in_link) + 1;
    gin = p.xprod + bd * p.nU + in_link;
    rin = p.xring + ((int64_t)bd * (p.nU - 1) + in_link) * p.xns * 16;
  }
  if (out_link >= 0) {
    out_next = first(out_link);
    out_end = last(out_link) + 1;
    gout = p.xprod + bd * p.nU + out_link;
    rout = p.xring + ((int64_t)bd * (p.nU - 1) + out_link) * p.xns * 16;
  }
  int idle = 0;
  while (in_next < in_end || out_next < out_end) {
    bool moved = false;
    if (in_next < in_end) {
      const int pub = __builtin_amdgcn_readfirstlane(xload_i32(gin));
      const int avail = min(min(pub, in_end), link_load(&g_link.cons[0]) + kLinkRing);
      if (avail > in_next) {
        const int n = min(avail - in_next, 64);
        if (lane < n) {  // the loads follow the progress load they depend on
          const int sq = in_next + lane;
          const double v = xload_f64((const double*)(rin + (int64_t)sq * 16));
          const int e = xload_i32((const int*)(rin + (int64_t)sq * 16 + 8));
          TDT_LDS volatile LinkSlot* sl = link_slot(0, sq);
          sl->v = v;
          sl->e = e;
        }
        in_next += n;
        link_store(&g_link.prod[0], in_next);
        moved = true;
      }
    }
    if (out_next < out_end) {
      const int avail = min(link_load(&g_link.prod[1]), out_end);
      if (avail > out_next) {
        const int n = min(avail - out_next, 64);
        if (lane < n) {
          const int sq = out_next + lane;
          TDT_LDS volatile LinkSlot* sl = link_slot(1, sq);
          xstore_f64((double*)(rout + (int64_t)sq * 16), sl->v);
          xstore_i32((int*)(rout + (int64_t)sq * 16 + 8), sl->e);
        }
        out_next += n;
        // every slot store complete before the progress store
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0) xstore_i32(gout, out_next);
        link_store(&g_link.cons[1], out_next);
        moved = true;
      }
    }
    if (moved) {
      idle = 0;
    } else {
      if (++idle > p.spin) return false;
      __builtin_amdgcn_s_sleep(2);
    }
  }
  return true;
}

// Long label sequences: one work-group of two waves per (utterance, direction, column of
// 64 labels over every frame), launched only when the GPU holds all of them at once (so a
// column never waits for a neighbour that has not started; the waits are bounded anyway).
// Wave 0 sweeps the column as a wave of k_tiles_link does, through LDS links (ring 0 in,
// ring 1 out); wave 1 carries those links to the neighbouring columns' work-groups
// (column_bridge), so the columns run at once, each behind its producer by about 64
// diagonals plus the bridge, and the utterance takes about T + U steps instead of one
// launch per band of tiles.  A column whose plain sweep went out of range, or whose links stalled, flags its
// (utterance, direction); the last of the columns to finish redoes it in extended range,
// strip after strip, and for beta finishes the utterance.  Extra work-groups zero the
// gradient's padding rows (as in k_tiles).  The tiles hold every frame (p.TT = Tmax).
__shared__ int g_col_last;
template <int DM>
__global__ __launch_bounds__(128) void k_cols(const Params p) {
  LinkShared& sh = g_link;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const uint32_t col_blocks = 2u * (uint32_t)p.B * (uint32_t)p.nU;
  if (blockIdx.x >= col_blocks) {
    zero_padded_rows(p, (blockIdx.x - col_blocks) * 2 + w, (gridDim.x - col_blocks) * 2, lane);
    return;
  }
  const int j = (int)(blockIdx.x % (uint32_t)p.nU), rest = (int)(blockIdx.x / (uint32_t)p.nU);
  const int dir = rest & 1, b = rest >> 1;
  const int64_t T64 = p.Tlen[b], U64 = p.Ulen[b];
  const bool dims = utt_dims_ok(p, T64, U64);
  const int T = dims ? (int)T64 : 0, U = dims ? (int)U64 : 0;
  const int ncol = dims ? U / 64 + 1 : 1;  // column 0 finishes an utterance with bad lengths
  if (j >= ncol) return;
  XCtl* ctl = p.xctl + (b * 2 + dir);
  Tile tl;
  const bool have = dims && make_tile(p, b, T, U, 0, j, 64, tl);
  const bool plain = have && p.pw && !p.xflag[b];
  if (threadIdx.x == 0) {
    sh.redo = 0;
    for (int i = 0; i < 2; ++i) {
      // ring 0: the link read, ring 1: the link written (i: its lower column)
      const int li = i == 0 ? (dir == 0 ? j - 1 : j) : (dir == 0 ? j : j - 1);
      sh.prod[i] = -(1 << 30);
      sh.cons[i] = dir == 0 ? 64 * (li + 1) - 1 : U - min(64 * li + 63, U);
    }
  }
  __syncthreads();
  Ext P = ext_zero();
  bool redo = false;
  if (w == 0) {
    if (have) {
      redo = true;
      if constexpr (plain_buffers<DM, 1>() >= 2) {
        if (plain) {
          LinkCtx lk{-1, -1, 0, 0, p.spin};
          if (dir == 0) {
            lk.in = j > 0 ? 0 : -1;
            lk.out = j + 1 < ncol ? 1 : -1;
            lk.in_last = T + tl.u0 - 2;
            redo = alpha_plain<DM, 1, false, true>(p, tl, lane, lk);
          } else {
            lk.in = j + 1 < ncol ? 0 : -1;
            lk.out = j > 0 ? 1 : -1;
            lk.in_last = T + U - (tl.u0 + 64);
            redo = beta_plain<DM, 1, false, true>(p, tl, lane, &P, lk);
          }
          redo = redo || lk.broken;
        }
      }
    }
  } else if (plain) {
    redo = !column_bridge(p, b, dir, j, ncol, T, U, lane);
  }
  if (__any(redo) && lane == 0) __hip_atomic_store(&sh.redo, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __syncthreads();
  if (threadIdx.x == 0) {  // (lane 0 of wave 0: it holds beta(0, 0) of column 0)
    if (sh.redo) __hip_atomic_fetch_or(&ctl->redo, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (dir == 1 && j == 0) {
      xstore_f64(&ctl->pm, P.m);
      xstore_i32(&ctl->pe, P.e);
    }
    // release: this column's records and words before the count; acquire: the last one
    // sees every column's
    const int old = __hip_atomic_fetch_add(&ctl->done, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const int lastc = old == ncol - 1 ? 1 : 0;
    g_col_last = lastc | (lastc && xload_i32(&ctl->redo) ? 2 : 0);
  }
  __syncthreads();
  const int fin = g_col_last;
  if (!(fin & 1) || w != 0) return;
  if (fin & 2) {
    // extended range, 64-label strips in dependency order (as in k_tiles_link)
    for (int s2 = 0; s2 < ncol; ++s2) {
      const int sj = dir == 0 ? s2 : ncol - 1 - s2;
      Tile st;
      if (!make_tile(p, b, T, U, 0, sj, 64, st)) continue;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (dir == 0) alpha_ext<DM>(p, st, lane);
      else beta_ext<DM>(p, st, lane, &P);
    }
  } else if (dir == 1) {
    P = Ext{xload_f64(&ctl->pm), xload_i32(&ctl->pe)};
  }
  if (dir == 1) finish_utterance(p, b, P, lane);
}

// ------------------------------------------------------------------------------------
// Posteriors and the per-node record of the long-row gradient pass (the short-row gradient
// pass computes the same numbers itself, a quarter wave per node: node_grad):
//   gamma(e) = alpha(n) W(e) beta(dest e) / P,   O(n) = sum over moves out of n,
//   c_blank, c_label = sums over blank / label moves, c_dur(d) = moves of duration d,
//   grad h_blank = w (O softmax(h)_blank - c_blank), grad h_y = w (O softmax(h)_y - c_label),
//   grad g_d = w (O softmax(g)_d - c_dur(d)),  other columns w O softmax(h)_v (streamed).

// One lane per position of the padded box (as in the node weights).  Utterances whose
// move weights all lie in [2^-300, 2^300] read the plain weights the lattice read; the
// others rebuild each weight in extended range from its ingredients.  The first
// work-group also reduces the loss (the lattice has finished every log P) unless the call
// writes no loss.  An upstream gradient (chain rule) scales w_b.  The record of the
// gradient pass overwrites the node's log-domain ingredients.
template <int DM>
__global__ __launch_bounds__(256) void k_coef(const Params p) {
  if (p.loss && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) reduce_loss(p);
  const int q = (int)(blockIdx.x * 256 + threadIdx.x);
  if (q >= p.box) return;
  int k, i;
  box_pos(p, q, k, i);
  const int u = diag_ulo(p, k) + i, t = k - u;
  const int len = diag_len(p, k);
  for (int b = blockIdx.y; b < p.B; b += gridDim.y) {
    // the per-utterance words (an ok utterance has valid lengths)
    const int ok = p.uok[b];
    const int T = (int)p.Tlen[b], U = (int)p.Ulen[b];
    if (!ok) continue;
    if (t >= T || u > U) continue;
    const int64_t pos = (int64_t)b * p.box + q;
    const bool plain = p.pw != nullptr && p.xflag[b] == 0;

    const Ext a = xrec_get(p.ar, pos);
    double* lgp = p.lg + pos * p.LG;
    const double lb = lgp[0], ly = lgp[1];
    double lam[DM + 1];
#pragma unroll
    for (int d = 0; d <= DM; ++d) lam[d] = p.didx[d] >= 0 ? lgp[2 + p.didx[d]] : -__builtin_inf();
    const double rP = 1.0 / p.pm[b];
    const int Pe = p.pe[b];
    const double* pw = plain ? p.pw + ((int64_t)b * pw_utt_entries(p.NP, p.box, p.KD) +
                                       (int64_t)p.NP * (q - i + 3 * (int64_t)k) + pw_col(i, len, p.R)) * 2
                             : nullptr;
    const int64_t pstride = (int64_t)(len + 3) * 2;  // doubles between slot pairs
    // posteriors of the blank / label move of each duration
    double cd[DM + 1];
    double cb = 0.0, cl = 0.0;
#pragma unroll
    for (int d = 0; d <= DM; ++d) {
      double gb = 0.0, gy = 0.0;
      if (p.didx[d] >= 0) {
        if (d >= 1) {
          Ext bt = ext_zero();
          if (t + d < T) bt = xrec_get(p.br, node_pos(p, b, t + d, u));
          else if (t + d == T && u == U) bt = ext_one();
          // the plain weight is loaded whether or not the destination holds a beta, so that
          // the loads of a node issue together
          const int sl = d - 1;
          const double wp = plain ? pw[(sl >> 1) * pstride + (sl & 1)] : 0.0;
          if (bt.m != 0.0) {
            const Ext w = plain ? Ext{wp, 0} : ext_exp(lb + lam[d]);
            gb = ext_to_double(Ext{a.m * w.m * bt.m * rP, a.e + w.e + bt.e - Pe});
          }
        }
        {
          const int sl = DM + d;
          const double wp = plain ? pw[(sl >> 1) * pstride + (sl & 1)] : 0.0;
          if (u < U && t + d < T) {
            const Ext bt = xrec_get(p.br, node_pos(p, b, t + d, u + 1));
            if (bt.m != 0.0) {
              const Ext w = plain ? Ext{wp, 0} : ext_exp(ly + lam[d]);
              gy = ext_to_double(Ext{a.m * w.m * bt.m * rP, a.e + w.e + bt.e - Pe});
            }
          }
        }
      }
      cd[d] = gb + gy;
      cb += gb;
      cl += gy;
    }
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
    float* rec = (float*)lgp;  // the ingredients have all been read above
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
    // softmax(g)_d and the duration gradients
#pragma unroll
    for (int d = 0; d <= DM; ++d)
      if (p.didx[d] >= 0) rec[5 + p.didx[d]] = (float)(wgt * (O * exp(lam[d]) - cd[d]));
  }
}

__global__ void k_reduce(const Params p) {
  if (threadIdx.x == 0) reduce_loss(p);
}

// ------------------------------------------------------------------------------------
// Launchers
// Work-groups of k_cols<DM> that the GPU running `st` holds at once (0 when unknown),
// from the occupancy of one CU times the CUs; kept per device.
template <int DM>
static int col_capacity(hipStream_t st) {
  constexpr int kDevices = 64;
  static int cache[kDevices] = {};
  int dev = -1;
  if (st ? hipStreamGetDevice(st, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= kDevices) return 0;
  int cap = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (cap == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_cols<DM>, 128, 0) != hipSuccess)
      return 0;
    cap = cus * per;
    __atomic_store_n(&cache[dev], cap, __ATOMIC_RELAXED);
  }
  return cap;
}

template <int DM>
static hipError_t launch_bands(const Params& p, hipStream_t st) {
  if (p.link) {
    const int zb = (p.zrows + p.nU - 1) / p.nU;  // zeroing waves, nU per work-group
    hipLaunchKernelGGL((k_tiles_link<DM>), dim3((unsigned)(2 * p.B + zb)), dim3(64 * p.nU), 0, st, p);
    return hipGetLastError();
  }
  if constexpr (plain_buffers<DM, 1>() >= 2) {
    if (p.xns) {  // linked columns, when every work-group can be resident at once
      const int zb = (p.zrows + 1) / 2;  // zeroing waves, two per work-group
      const int grid = 2 * p.B * p.nU + zb;
      if (grid <= col_capacity<DM>(st)) {
        Params q = p;
        q.TT = p.Tmax;
        q.nT = 1;
        hipLaunchKernelGGL((k_cols<DM>), dim3((unsigned)grid), dim3(128), 0, st, q);
        return hipGetLastError();
      }
    }
  }
  const bool banded = p.nT > 1 || p.nU > 1;
  for (int band = 0; band < p.nT + p.nU - 1; ++band) {
    const int ilo = band - (p.nU - 1) > 0 ? band - (p.nU - 1) : 0;
    const int ihi = band < p.nT - 1 ? band : p.nT - 1;
    const dim3 grid((unsigned)((ihi - ilo + 1) * 2 * p.B + (band == 0 ? p.zrows : 0)));
    if (banded) hipLaunchKernelGGL((k_tiles<DM, 1, true>), grid, dim3(64), 0, st, p, band);
    else hipLaunchKernelGGL((k_tiles<DM, 1, false>), grid, dim3(64), 0, st, p, band);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_lattice_side(const Params& p, int which, hipStream_t st) {
  // one lane per node: [positions of the padded box, utterances]
  const dim3 gridg((unsigned)((p.box + 255) / 256), (unsigned)(p.B < 65535 ? p.B : 65535));
  switch (which) {
    case 0:  // node weights
      if (p.DM == 4) hipLaunchKernelGGL((k_node_weights<4>), gridg, dim3(256), 0, st, p);
      else if (p.DM == 8) hipLaunchKernelGGL((k_node_weights<8>), gridg, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((k_node_weights<16>), gridg, dim3(256), 0, st, p);
      return hipGetLastError();
    case 1:  // lattice: the bands of tiles
      if (p.DM == 4) return launch_bands<4>(p, st);
      if (p.DM == 8) return launch_bands<8>(p, st);
      return launch_bands<16>(p, st);
    case 2:  // coefficients (and the loss reduction)
      if (p.DM == 4) hipLaunchKernelGGL((k_coef<4>), gridg, dim3(256), 0, st, p);
      else if (p.DM == 8) hipLaunchKernelGGL((k_coef<8>), gridg, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((k_coef<16>), gridg, dim3(256), 0, st, p);
      return hipGetLastError();
    default:  // loss reduction over the whole batch
      hipLaunchKernelGGL(k_reduce, dim3(1), dim3(64), 0, st, p);
      return hipGetLastError();
  }
}

}  // namespace tdt
