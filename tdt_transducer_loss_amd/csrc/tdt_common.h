// Shared definitions of the gfx950 TDT loss kernels: launch parameters, the workspace
// layout, extended-range float64 arithmetic and element-type traits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tdt {

constexpr int kWave = 64;
constexpr int kMaxD = 16;      // durations per call
constexpr int kMaxDval = 16;   // largest duration value
constexpr int kEZ = -(1 << 28);  // exponent of the extended-range zero
// Stored weight exponents carry this bias, so a weight read as all-zero bits (out of
// range of a buffer load) decodes as mantissa 0 with exponent -kWBias: a zero.
constexpr int kWBias = 1 << 29;

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2 = 0.6931471805599453094;
constexpr double kLn2Hi = 6.93147180369123816490e-01;  // ln2 with 32 trailing zero bits
constexpr double kLn2Lo = 1.90821492927058770002e-10;
constexpr double kLog2eD = 1.4426950408889634074;

// Division of a non-negative int below 2^31 by a fixed divisor d:
//   n / d = (mulhi(n, m) + n) >> s,  s = ceil(log2 d),  m = floor(2^32 (2^s - d) / d) + 1
// (Granlund and Montgomery, "Division by invariant integers using multiplication",
// PLDI 1994; the add cannot overflow for n < 2^31).
struct FastDiv {
  uint32_t m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while (((uint64_t)1 << s) < d) ++s;
  const uint64_t m = (((uint64_t)1 << 32) * (((uint64_t)1 << s) - d)) / d + 1;
  return FastDiv{(uint32_t)m, s};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) { return (__umulhi(n, f.m) + n) >> f.s; }

// Everything the kernels of one call need, passed by value.
//
// Workspace layout.  Per utterance b the nodes (t, u) of the padded box
// [0, Tmax) x [0, U1max) are stored diagonal-major: diagonal k = t + u in [0, KD), and
// within it by u, so node (t, u) sits at
//   pos = b * box + diag_off(k) + u - max(0, k - Tmax + 1),   box = Tmax * U1max,
// where diag_off(k) counts the box nodes on diagonals below k (closed form below).  One
// step of a lattice sweep (one anti-diagonal) thus reads and writes consecutive records,
// and the workspace holds exactly the padded box (nodes outside an utterance are unused).
struct Params {
  int B, Tmax, U1max, V, D, blank, red, dtype;
  int KD;            // diagonals of the padded box: Tmax + U1max - 1
  int A, Bb;         // min and max of Tmax, U1max
  int64_t box;       // Tmax * U1max
  int64_t triA;      // A (A + 1) / 2
  int DM, NW, NP;    // duration bound of the kernels, move slots 2 DM + 1, slot pairs DM + 1
  int LG;            // doubles per node in lg: 2 + D
  int RS;            // floats of the gradient-pass record: 5 + D
  int R;             // labels per lane of the lattice sweep (1)
  int nT, nU, TT;    // lattice tiles: nT rows of TT frames, nU columns of 64 R labels
  int link;          // 1: one work-group of nU waves sweeps an utterance's nU label tiles at once
  int xns;           // > 0: label columns linked across work-groups are possible (cross-column
                     //   workspace present); slots per link ring
  int nseg, nch;     // row-statistics pass: segments per row, 64-chunk windows per segment
  int gnseg, gnch;   // the same for the gradient pass
  FastDiv fd_nseg, fd_gnseg, fd_u1, fd_tu1, fd_a;  // by nseg, gnseg, U1max, Tmax*U1max, A
  double sigma;
  int dval[kMaxD];          // duration value of index i
  int didx[kMaxDval + 1];   // index of duration value d, -1 when absent
  // inputs (element strides of the first three dims; last dim contiguous)
  const void* tok;
  int64_t ts0, ts1, ts2;
  const void* dur;
  int64_t ds0, ds1, ds2;
  const int64_t* labels;
  int64_t lab_stride;
  const int64_t* Tlen;
  const int64_t* Ulen;
  // outputs
  float* loss;     // NULL: the loss is not written (gradient-only call)
  int32_t* ustatus;
  const float* gscale;  // gradient scale per utterance ([B], reduction none) or [1]; NULL = 1
  void* gtok;
  int64_t gs0, gs1, gs2;
  void* gdur;
  int64_t gds0, gds1, gds2;
  // workspace, per node position
  float* part;    // [nseg] float2 per row segment: its shift c and its sum 2^(x log2e - c), see
                  //   k_row_partial; node-major order (b, t, u), unlike the other per-node
                  //   arrays, so that the row passes write consecutive rows' records together
  float2* stat;   // row statistics (c, K) written by the node weights, lse = row_lse(c, K)
  double* lg;     // [LG]: l_blank - sigma, l_label - sigma, lambda[D] (log-softmax of the
                  //   durations); the coefficient kernel overwrites it with the RS floats
                  //   of the gradient-pass record
  double* pw;     // plain outgoing move weights by slot pairs, see pw_entry
  char* ar;       // alpha, 16-byte records (float64 mantissa, int32 exponent)
  char* br;       // beta, same records
  char* lx;       // [b][nU][Tmax] 16-byte records: label contributions crossing a tile column edge
  // workspace, per utterance
  double* logp;   // log P from beta(0,0)
  double* wts;    // reduction weight w_b
  double* pm;     // P as mantissa / exponent
  int* pe;
  int* uok;       // 1: gradients are written from the lattice, 0: zeros
  int* xflag;     // 1: some move weight lies outside [2^-300, 2^300] (extended-range sweep only)
  // workspace of label columns linked across work-groups (when xns > 0), reset by the node
  // weights: per (utterance, direction) a control word, per (utterance, direction, column)
  // the progress of the link it writes, per (utterance, direction, link) a ring of xns
  // 16-byte slots
  struct XCtl* xctl;
  int* xprod;
  char* xring;
  // gradient rows outside every utterance's lattice (padding): 0 = written (zeros) by the
  // gradient pass; > 0 = zeroed by that many extra waves of the first lattice launch (they
  // overlap the sweeps) and skipped by the gradient pass
  int zrows;
  // 1: the short-row statistics read the logits with nontemporal loads (a padded batch of
  // more than twice the 256 MB last-level cache, whose reuse by the gradient pass is small)
  int rows_nt;
  // long-row statistics: the rows of nodes below nt_nodes (all but the last 256 MB of the
  // padded batch in memory order) are read with nontemporal loads, the rest with ordinary
  // ones, which leave them in the last-level cache for the gradient pass (it starts there)
  uint32_t nt_nodes;
  // iterations a wait between lattice waves or work-groups may take before it gives up and
  // the utterance is redone in extended range (2^20, about 0.1 s; the environment variable
  // TDT_LINK_SPIN_LIMIT lowers it, so that tests can force that path)
  int spin;
};

// bytes of the GPU's last-level cache (MI355X Infinity Cache)
constexpr double kLastLevelCacheBytes = 256.0 * 1024 * 1024;

// Column work-groups (2 B nU) up to which the workspace holds the links of long label
// sequences run as linked columns (the launch also checks that the GPU holds them all at
// once: about two to four two-wave work-groups per CU)
constexpr int kMaxColBlocks = 768;

// Control word of one (utterance, direction) of the linked columns: columns finished,
// a column asked for the extended-range redo, and beta(0, 0) from the first column.
struct XCtl {
  int done, redo, pe, pad;
  double pm;
};

// ---- padded-box diagonal layout ----
// box nodes on diagonals 0 .. k-1
__device__ __forceinline__ int64_t diag_off(const Params& p, int k) {
  if (k <= p.A) return (int64_t)k * (k + 1) / 2;
  if (k <= p.Bb) return p.triA + (int64_t)(k - p.A) * p.A;
  const int64_t r = p.KD - k;
  return p.box - r * (r + 1) / 2;
}
// smallest u on diagonal k, and the diagonal's node count
__device__ __forceinline__ int diag_ulo(const Params& p, int k) { return max(0, k - p.Tmax + 1); }
__device__ __forceinline__ int diag_len(const Params& p, int k) {
  return min(k, p.U1max - 1) - diag_ulo(p, k) + 1;
}
// largest k with k (k + 1) / 2 <= n, for 0 <= n < 2^27 (the float square root is off by
// less than one, so one correction step suffices)
__device__ __forceinline__ int tri_root(int n) {
  int k = (int)((sqrtf(8.f * (float)n + 1.f) - 1.f) * 0.5f);
  if ((k + 1) * (k + 2) / 2 <= n) ++k;
  else if (k * (k + 1) / 2 > n) --k;
  return k;
}
// Diagonal k and index i on it of position q in [0, box) of an utterance's padded box
// (the inverse of diag_off): diagonals 1 .. A long up to triA, then a band of A-long
// diagonals, then diagonals A - 1 .. 1 long.
__device__ __forceinline__ void box_pos(const Params& p, int q, int& k, int& i) {
  const int tri = (int)p.triA;
  const int tail0 = (int)(p.box - p.triA + p.A);
  if (q < tri) {
    k = tri_root(q);
    i = q - k * (k + 1) / 2;
  } else if (q < tail0) {
    const int r = q - tri;
    const int m = (int)fdiv((uint32_t)r, p.fd_a);
    k = p.A + m;
    i = r - m * p.A;
  } else {
    const int s = (int)(p.box - 1) - q;  // position counted from the box's last node
    const int kk = tri_root(s);
    k = p.KD - 1 - kk;
    i = kk - (s - kk * (kk + 1) / 2);
  }
}
// position of node (t, u) of utterance b
__device__ __forceinline__ int64_t node_pos(const Params& p, int b, int t, int u) {
  const int k = t + u;
  return (int64_t)b * p.box + diag_off(p, k) + (u - diag_ulo(p, k));
}
// Plain outgoing weights: per utterance, diagonal k owns a block of NP x (len(k) + 3)
// 16-byte entries at entry NP (diag_off(k) + 3k) (slot pairs major, one column per node
// of the diagonal, up to 3 unused columns); entry (pair q, node index i) is at column
// (i % R) * ceil(len / R) + i / R, so that the lanes of a sweep holding R labels each read
// consecutive entries for each of their labels.  Slot d - 1 (d = 1..DM) is the blank move
// of duration d, slot DM + d (d = 0..DM) the label move of duration d.
__host__ __device__ constexpr int64_t pw_utt_entries(int64_t NP, int64_t box, int64_t KD) {
  return NP * (box + 3 * KD);
}
__device__ __forceinline__ int64_t pw_block(const Params& p, int k) { return (int64_t)p.NP * (diag_off(p, k) + 3 * (int64_t)k); }
__device__ __forceinline__ int pw_col(int i, int len, int R) {
  const int half = (len + R - 1) / R;
  return R == 1 ? i : (i % R) * half + i / R;
}

// ---- extended-range non-negative numbers: value = m * 2^e ----
struct Ext {
  double m;
  int e;
};

__device__ __forceinline__ Ext ext_zero() { return Ext{0.0, kEZ}; }
__device__ __forceinline__ Ext ext_one() { return Ext{0.5, 1}; }
__device__ __forceinline__ Ext ext_mul(Ext a, Ext b) { return Ext{a.m * b.m, a.e + b.e}; }

// Normalise a sum s * 2^E to a mantissa in [0.5, 1).  Results below 2^-(2^27) are
// zero (as in ext_exp), so exponent sums of a sweep stay far inside the int range.
__device__ __forceinline__ Ext ext_norm(double s, int E) {
  if (s == 0.0) return ext_zero();
  int ex;
  double m = frexp(s, &ex);  // v_frexp_mant_f64 / v_frexp_exp_i32_f64
  return E + ex < -(1 << 27) ? ext_zero() : Ext{m, E + ex};
}

// exp(x) in extended range, accurate to a few ulp of float64.  The argument reduction
// x = k ln2 + r splits ln2 into a high part with trailing zero bits and a low part
// (Cody and Waite, "Software Manual for the Elementary Functions", 1980), so k ln2 is
// exact for the k that occur.  Values below 2^-(2^27) (x below about -9.3e7, e.g. a
// logit masked with -1e10) are taken as zero: their exponent would not fit the int
// exponent arithmetic of the sweeps.
__device__ __forceinline__ Ext ext_exp(double x) {
  if (!(x > -1.0e300)) {  // -inf (or a huge negative value): zero; NaN propagates below
    if (x != x) return Ext{x, 0};
    return ext_zero();
  }
  double kf = floor(x * kLog2eD);
  if (kf > 1.0e9) return Ext{__builtin_inf(), 0};
  if (kf < -(double)(1 << 27)) return ext_zero();
  int k = (int)kf;
  double r = fma(-kf, kLn2Hi, x);
  r = fma(-kf, kLn2Lo, r);
  return Ext{exp(r), k};
}

__device__ __forceinline__ double ext_log(Ext a) {
  if (a.m == 0.0) return -__builtin_inf();
  return log(a.m) + (double)a.e * kLn2;
}

__device__ __forceinline__ double ext_to_double(Ext a) {
  if (a.m == 0.0) return 0.0;
  int e = a.e;
  e = e < -2100 ? -2100 : (e > 2100 ? 2100 : e);
  return ldexp(a.m, e);
}

// alpha / beta record of a node, normalised (the plain sweeps store unnormalised values)
__device__ __forceinline__ Ext xrec_get(const char* base, int64_t pos) {
  const char* r = base + pos * 16;
  return ext_norm(*(const double*)r, *(const int*)(r + 8));
}

// The reduced loss from every utterance's log P and reduction weight (one thread).
__device__ inline void reduce_loss(const Params& p) {
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

// Sum of N extended values: align to the largest exponent, add, renormalise.
template <int N>
__device__ __forceinline__ Ext ext_sum(const Ext (&t)[N]) {
  int E = t[0].e;
#pragma unroll
  for (int i = 1; i < N; ++i) E = max(E, t[i].e);
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < N; ++i) s += ldexp(t[i].m, t[i].e - E);
  return ext_norm(s, E);
}

// Log-sum-exp of a row from its statistics {c, K}: 32-bit logits keep c as the row
// maximum (the sum is taken of 2^((x - c) log2e)), 16-bit logits keep c in base-2 units
// (the sum is taken of 2^(x log2e - c)); K = log2 of the sum.
__device__ __forceinline__ double row_lse(bool base2, double c, double K) {
  return base2 ? (c + K) * kLn2 : c + K * kLn2;
}

__device__ __forceinline__ bool utt_dims_ok(const Params& p, int64_t T, int64_t U) {
  return T >= 0 && T <= p.Tmax && U >= 0 && U <= p.U1max - 1;
}

// Work-groups are handed to the 8 XCDs round-robin; remap so that consecutive logical
// blocks (neighbouring lattice positions) share an XCD and its L2.
__device__ __forceinline__ uint32_t xcd_block(uint32_t g, uint32_t G) {
  constexpr uint32_t nx = 8;
  uint32_t q = G / nx, r = G % nx, x = g % nx, idx = g / nx;
  return x < r ? x * (q + 1) + idx : r * (q + 1) + (x - r) * q + idx;
}

// Global-memory (address space 1) pointers: accesses through them compile to global_*
// instructions.  Through generic pointers they are flat_* ones, which count on both
// memory counters, so that waiting for one of them waits for every access in flight.
#define TDT_GLOBAL __attribute__((address_space(1)))
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---- element types ----
struct F32 {
  using T = float;
  static constexpr int kEpc = 4;  // elements per 16-byte chunk
  static constexpr uint32_t kNegInf = 0xff800000u;
  __device__ static __forceinline__ float load(const void* p, int64_t i) { return ((const TDT_GLOBAL float*)p)[i]; }
  __device__ static __forceinline__ void store(void* p, int64_t i, float v) { ((TDT_GLOBAL float*)p)[i] = v; }
  __device__ static __forceinline__ float get(const uint4& c, int s) {
    uint32_t w = s == 0 ? c.x : s == 1 ? c.y : s == 2 ? c.z : c.w;
    return __uint_as_float(w);
  }
  // element s of a chunk, s a compile-time constant after unrolling
  template <int S>
  __device__ static __forceinline__ float at(const uint4& c) {
    return __uint_as_float(S == 0 ? c.x : S == 1 ? c.y : S == 2 ? c.z : c.w);
  }
  __device__ static __forceinline__ uint32_t bits(float v) { return __float_as_uint(v); }
  __device__ static __forceinline__ uint4 pack(const float (&v)[4]) {
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
  }
};

struct BF16 {
  using T = uint16_t;
  static constexpr int kEpc = 8;
  static constexpr uint32_t kNegInf = 0xff80u;
  __device__ static __forceinline__ float load(const void* p, int64_t i) {
    return __uint_as_float(((uint32_t)((const TDT_GLOBAL uint16_t*)p)[i]) << 16);
  }
  __device__ static __forceinline__ uint32_t bits(float v) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v);  // round to nearest even
  }
  __device__ static __forceinline__ void store(void* p, int64_t i, float v) { ((TDT_GLOBAL uint16_t*)p)[i] = (uint16_t)bits(v); }
  __device__ static __forceinline__ float get(const uint4& c, int s) {
    uint32_t w = (s >> 1) == 0 ? c.x : (s >> 1) == 1 ? c.y : (s >> 1) == 2 ? c.z : c.w;
    return __uint_as_float((s & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  template <int S>
  __device__ static __forceinline__ float at(const uint4& c) {
    uint32_t w = (S >> 1) == 0 ? c.x : (S >> 1) == 1 ? c.y : (S >> 1) == 2 ? c.z : c.w;
    return __uint_as_float((S & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    f2 in = {lo, hi};
    bf2 out = __builtin_convertvector(in, bf2);  // v_cvt_pk_bf16_f32, round to nearest even
    return __builtin_bit_cast(uint32_t, out);
  }
  __device__ static __forceinline__ uint4 pack(const float (&v)[8]) {
    return make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7]));
  }
};

struct F16 {
  using T = uint16_t;
  static constexpr int kEpc = 8;
  static constexpr uint32_t kNegInf = 0xfc00u;
  __device__ static __forceinline__ float h2f(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }
  __device__ static __forceinline__ float load(const void* p, int64_t i) { return h2f(((const TDT_GLOBAL uint16_t*)p)[i]); }
  __device__ static __forceinline__ uint32_t bits(float v) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);  // round to nearest even
  }
  __device__ static __forceinline__ void store(void* p, int64_t i, float v) { ((TDT_GLOBAL uint16_t*)p)[i] = (uint16_t)bits(v); }
  __device__ static __forceinline__ float get(const uint4& c, int s) {
    uint32_t w = (s >> 1) == 0 ? c.x : (s >> 1) == 1 ? c.y : (s >> 1) == 2 ? c.z : c.w;
    return h2f((s & 1) ? (w >> 16) : (w & 0xffffu));
  }
  template <int S>
  __device__ static __forceinline__ float at(const uint4& c) {
    uint32_t w = (S >> 1) == 0 ? c.x : (S >> 1) == 1 ? c.y : (S >> 1) == 2 ? c.z : c.w;
    return h2f((S & 1) ? (w >> 16) : (w & 0xffffu));
  }
  __device__ static __forceinline__ uint32_t pack2(float lo, float hi) { return bits(lo) | (bits(hi) << 16); }
  __device__ static __forceinline__ uint4 pack(const float (&v)[8]) {
    return make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7]));
  }
};

// Replace element s of a chunk by the pattern `bitsv` (element width from TI).
template <typename TI>
__device__ __forceinline__ void chunk_set(uint4& c, int s, uint32_t bitsv) {
  if (TI::kEpc == 4) {
    if (s == 0) c.x = bitsv;
    else if (s == 1) c.y = bitsv;
    else if (s == 2) c.z = bitsv;
    else c.w = bitsv;
  } else {
    const int w = s >> 1;
    const uint32_t sh = (s & 1) ? 16u : 0u;
    const uint32_t keep = ~(0xffffu << sh);
    const uint32_t put = (bitsv & 0xffffu) << sh;
    if (w == 0) c.x = (c.x & keep) | put;
    else if (w == 1) c.y = (c.y & keep) | put;
    else if (w == 2) c.z = (c.z & keep) | put;
    else c.w = (c.w & keep) | put;
  }
}

// ---- wave reductions (64 lanes) ----
// DPP forms: quad swaps, then the half-row and row mirrors leave every lane of a 16-lane
// row holding the row's result; the four rows are combined from lanes 0, 16, 32, 48.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(x)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const long long b = __double_as_longlong(x);
  const int lo = dpp_i<CTRL>((int)b), hi = dpp_i<CTRL>((int)(b >> 32));
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}
__device__ __forceinline__ float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ double readlane_d(double x, int l) {
  const long long b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_readlane((int)b, l), hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}
// maximum over the wave, uniform result
__device__ __forceinline__ float wave_max_dpp(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_f<0x140>(x));  // row_mirror
  return fmaxf(fmaxf(readlane_f(x, 0), readlane_f(x, 16)), fmaxf(readlane_f(x, 32), readlane_f(x, 48)));
}
// sum over the wave, uniform result (a fixed order: deterministic)
__device__ __forceinline__ double wave_sum_dpp(double x) {
  x += dpp_d<0xB1>(x);
  x += dpp_d<0x4E>(x);
  x += dpp_d<0x141>(x);
  x += dpp_d<0x140>(x);
  return (readlane_d(x, 0) + readlane_d(x, 16)) + (readlane_d(x, 32) + readlane_d(x, 48));
}

__device__ __forceinline__ float wave_max_f32(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

}  // namespace tdt
