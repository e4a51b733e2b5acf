// Host side of the C ABI declared in include/tdt_loss.h: argument validation, workspace
// layout and the launch sequence.  On the caller's stream the kernels run
//   row partials -> node weights -> lattice (alpha || beta) -> coefficients and loss
//   reduction -> gradient  (short rows: the gradient pass computes the coefficients and
//   reduces the loss itself; forward only: ... -> lattice -> loss reduction; a later
//   backward call on the same workspace: [coefficients ->] gradient).
#include <algorithm>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "tdt_kernels.h"
#include "tdt_loss.h"
#include "tdt_rows.h"

namespace {

using tdt::Params;

struct Layout {
  int KD, A, Bb, DM, NW, NP, LG, RS, R, nT, nU, TT, link, xns, nseg, nch, gnseg, gnch;
  int64_t box;
  size_t pw_bytes;
  size_t off_part, off_stat, off_lg, off_pw, off_ar, off_br, off_lx;
  size_t off_logp, off_wts, off_pm, off_pe, off_uok, off_xflag, off_xctl, off_xprod, off_xring;
  size_t total;
};

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

int pick_dm(int maxd) { return maxd <= 4 ? 4 : (maxd <= 8 ? 8 : 16); }

// Validate the duration list and return its largest value (or a negative code).
int check_durations(const int32_t* durations, int32_t D) {
  if (!durations || D < 1) return TDT_ERR_INVALID_ARGUMENT;
  if (D > TDT_MAX_DURATIONS) return TDT_ERR_UNSUPPORTED;
  int maxd = -1;
  bool any_pos = false;
  for (int i = 0; i < D; ++i) {
    const int d = durations[i];
    if (d < 0) return TDT_ERR_INVALID_ARGUMENT;
    if (d > TDT_MAX_DURATION_VALUE) return TDT_ERR_UNSUPPORTED;
    for (int j = 0; j < i; ++j)
      if (durations[j] == d) return TDT_ERR_INVALID_ARGUMENT;
    any_pos |= d > 0;
    maxd = d > maxd ? d : maxd;
  }
  return any_pos ? maxd : TDT_ERR_INVALID_ARGUMENT;
}

// Workspace layout (every array 256-byte aligned), per node position of the padded box
// [B, Tmax, U1max] in diagonal-major order (see Params): row-segment partials, row
// statistics, log-domain move ingredients (overwritten by the gradient-pass record),
// plain outgoing weights, alpha and beta; per utterance and tile column the label
// contributions crossing a tile edge; per utterance a few words.
int make_layout(int32_t dtype, int64_t B, int64_t Tmax, int64_t U1max, int64_t V, int32_t D, int maxd, Layout* L) {
  if (dtype < 0 || dtype > 2) return TDT_ERR_UNSUPPORTED_DTYPE;
  if (B < 1 || Tmax < 1 || U1max < 1 || V < 1) return TDT_ERR_INVALID_ARGUMENT;
  if (V > ((int64_t)1 << 30) || B > ((int64_t)1 << 24)) return TDT_ERR_UNSUPPORTED;
  if (Tmax > (1 << 24) || U1max > (1 << 24)) return TDT_ERR_UNSUPPORTED;
  L->box = Tmax * U1max;
  // alpha / beta / edge records of one utterance are addressed with 32-bit byte offsets
  if (L->box * 16 >= ((int64_t)1 << 31)) return TDT_ERR_UNSUPPORTED;
  L->KD = (int)(Tmax + U1max - 1);
  L->A = (int)(Tmax < U1max ? Tmax : U1max);
  L->Bb = (int)(Tmax < U1max ? U1max : Tmax);
  L->DM = pick_dm(maxd);
  L->NW = 2 * L->DM + 1;
  L->NP = L->DM + 1;
  L->LG = 2 + D;
  L->RS = 5 + D;
  // lattice tiles of 64 labels (one per lane): up to 256 labels, tiles holding every frame
  // swept at once by the waves of one work-group (linked through LDS); longer label
  // sequences, columns of 64 labels and every frame in work-groups of their own, linked
  // through global memory (durations up to 8 and at most kMaxColBlocks work-groups), else
  // bands of 64-label x 48-frame tiles (B2 T1000 U1500 durations 0..8: 32 / 40 / 48 / 64 /
  // 96 / 128 frames, lattice 3.42 / 3.25 / 3.06 / 3.14 / 3.26 / 3.55 ms)
  L->R = 1;
  L->xns = 0;
  if (U1max <= 256) {
    L->TT = (int)Tmax;
    L->nT = 1;
    L->nU = (int)((U1max + 63) / 64);
    L->link = L->nU > 1 ? 1 : 0;
  } else {
    L->TT = 48;
    L->nT = (int)((Tmax + 47) / 48);
    L->nU = (int)((U1max + 63) / 64);
    L->link = 0;
    if (L->DM <= 8 && 2 * B * L->nU <= tdt::kMaxColBlocks) L->xns = (int)(Tmax + U1max + 64);
  }
  // a row's chunks: from its own 16-byte chunk (row statistics, one more chunk than V
  // fills) or from its 128-byte line (gradient pass, up to 8 more)
  tdt::pick_segments(V, dtype == 0 ? 4 : 8, tdt::kRowWindows, 1, &L->nch, &L->nseg);
  tdt::pick_segments(V, dtype == 0 ? 4 : 8, tdt::kGradWindows, 8, &L->gnch, &L->gnseg);
  const size_t NPOS = (size_t)B * (size_t)L->box;
  // the row passes index (node, row segment) pairs with 32-bit integers
  const size_t segs = (size_t)(L->nseg > L->gnseg ? L->nseg : L->gnseg);
  if (NPOS * segs >= ((size_t)1 << 31)) return TDT_ERR_UNSUPPORTED;
  const size_t nu64 = (size_t)((U1max + 63) / 64);
  if (nu64 * (size_t)Tmax * 16 >= ((size_t)1 << 31)) return TDT_ERR_UNSUPPORTED;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L->off_part = take(NPOS * (size_t)L->nseg * 8);
  L->off_stat = take(NPOS * 8);
  L->off_lg = take(NPOS * (size_t)L->LG * 8);
  // plain weights, addressed with 32-bit byte offsets per utterance (without them the
  // extended-range sweeps run)
  const size_t pw_utt = (size_t)tdt::pw_utt_entries(L->NP, L->box, L->KD) * 16;
  L->pw_bytes = pw_utt < ((size_t)1 << 31) ? pw_utt * (size_t)B : 0;
  L->off_pw = take(L->pw_bytes);
  L->off_ar = take(NPOS * 16);
  L->off_br = take(NPOS * 16);
  L->off_lx = take((size_t)B * nu64 * (size_t)Tmax * 16);
  L->off_logp = take((size_t)B * 8);
  L->off_wts = take((size_t)B * 8);
  L->off_pm = take((size_t)B * 8);
  L->off_pe = take((size_t)B * 4);
  L->off_uok = take((size_t)B * 4);
  L->off_xflag = take((size_t)B * 4);
  L->off_xctl = take(L->xns ? (size_t)B * 2 * sizeof(tdt::XCtl) : 0);
  L->off_xprod = take(L->xns ? (size_t)B * 2 * (size_t)L->nU * 4 : 0);
  L->off_xring = take(L->xns ? (size_t)B * 2 * (size_t)(L->nU - 1) * (size_t)L->xns * 16 : 0);
  L->total = o;
  return TDT_OK;
}

bool aligned_to(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

}  // namespace

extern "C" int tdt_loss_abi_version(void) { return 3; }

extern "C" const char* tdt_loss_status_string(int status) {
  switch (status) {
    case TDT_OK: return "ok";
    case TDT_ERR_INVALID_ARGUMENT: return "invalid argument";
    case TDT_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case TDT_ERR_BAD_STRIDE: return "bad stride or misaligned pointer";
    case TDT_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case TDT_ERR_UNSUPPORTED: return "size beyond the limits of this library";
    case TDT_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

extern "C" int tdt_loss_workspace_size(int32_t dtype, int64_t B, int64_t T_max, int64_t U1_max, int64_t V,
                                       const int32_t* durations, int32_t num_durations, size_t* bytes) {
  if (!bytes) return TDT_ERR_INVALID_ARGUMENT;
  const int maxd = check_durations(durations, num_durations);
  if (maxd < 0) return maxd;
  Layout L;
  const int rc = make_layout(dtype, B, T_max, U1_max, V, num_durations, maxd, &L);
  if (rc != TDT_OK) return rc;
  *bytes = L.total;
  return TDT_OK;
}

namespace {

// Byte range [lo, hi) touched by a [B, T, U1, C] view with element strides s[0..2] and a
// unit last stride.
struct Extent {
  __int128 lo, hi;
};

Extent view_extent(const void* ptr, const int64_t* s, int64_t B, int64_t T, int64_t U1, int64_t C, size_t elt) {
  const int64_t n[3] = {B, T, U1};
  __int128 lo = 0, hi = C;
  for (int d = 0; d < 3; ++d) {
    const __int128 off = (__int128)(n[d] - 1) * s[d];
    if (off < 0) lo += off;
    else hi += off;
  }
  const __int128 base = (__int128)(uintptr_t)ptr;
  return Extent{base + lo * (__int128)elt, base + hi * (__int128)elt};
}

bool overlap(const Extent& a, const Extent& b) { return a.lo < b.hi && b.lo < a.hi; }

bool same_view(const void* a, const int64_t* sa, const void* b, const int64_t* sb) {
  return a == b && sa[0] == sb[0] && sa[1] == sb[1] && sa[2] == sb[2];
}

// Validates the arguments shared by every entry point and fills the kernel parameters.
// `grads`: gradient views are given (required when need_grads).
int prepare(int32_t dtype, int64_t B, int64_t T_max, int64_t U1_max, int64_t V, const void* logits,
            const int64_t* logits_strides, const void* dur_logits, const int64_t* dur_strides, int32_t num_durations,
            const int64_t* labels, int64_t labels_stride, const int64_t* logit_lengths, const int64_t* label_lengths,
            const int32_t* durations, int32_t blank, double sigma, int32_t reduction, float* loss_out,
            bool need_loss, bool need_grads, void* grad_logits, const int64_t* grad_strides, void* grad_dur_logits,
            const int64_t* grad_dur_strides, int32_t* utt_status, void* workspace, size_t workspace_bytes,
            Params* pp, bool* grads_out, bool* aligned_out) {
  if (dtype < 0 || dtype > 2) return TDT_ERR_UNSUPPORTED_DTYPE;
  if (reduction < 0 || reduction > 4) return TDT_ERR_INVALID_ARGUMENT;
  if (!logits || !logits_strides || !dur_logits || !dur_strides || !labels || !logit_lengths || !label_lengths ||
      !workspace)
    return TDT_ERR_INVALID_ARGUMENT;
  if (need_loss && !loss_out) return TDT_ERR_INVALID_ARGUMENT;
  if (V < 1) return TDT_ERR_INVALID_ARGUMENT;
  if (blank < 0 || blank >= V) return TDT_ERR_INVALID_ARGUMENT;
  if (!isfinite(sigma)) return TDT_ERR_INVALID_ARGUMENT;
  if (labels_stride < U1_max - 1) return TDT_ERR_BAD_STRIDE;
  const bool grads = grad_logits != nullptr || grad_dur_logits != nullptr;
  if (grads && (!grad_logits || !grad_dur_logits || !grad_strides || !grad_dur_strides))
    return TDT_ERR_INVALID_ARGUMENT;
  if (need_grads && !grads) return TDT_ERR_INVALID_ARGUMENT;
  const int maxd = check_durations(durations, num_durations);
  if (maxd < 0) return maxd;
  Layout L;
  int rc = make_layout(dtype, B, T_max, U1_max, V, num_durations, maxd, &L);
  if (rc != TDT_OK) return rc;
  const size_t elt = dtype == 0 ? 4 : 2;
  if (grads) {
    // a gradient view is either exactly its logits view (in place) or disjoint from both
    // logits views
    const Extent et = view_extent(logits, logits_strides, B, T_max, U1_max, V, elt);
    const Extent ed = view_extent(dur_logits, dur_strides, B, T_max, U1_max, num_durations, elt);
    if (!same_view(grad_logits, grad_strides, logits, logits_strides)) {
      const Extent eg = view_extent(grad_logits, grad_strides, B, T_max, U1_max, V, elt);
      if (overlap(eg, et) || overlap(eg, ed)) return TDT_ERR_INVALID_ARGUMENT;
    }
    if (!same_view(grad_dur_logits, grad_dur_strides, dur_logits, dur_strides)) {
      const Extent eg = view_extent(grad_dur_logits, grad_dur_strides, B, T_max, U1_max, num_durations, elt);
      if (overlap(eg, et) || overlap(eg, ed)) return TDT_ERR_INVALID_ARGUMENT;
    }
  }
  if (workspace_bytes < L.total) return TDT_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned_to(workspace, 256)) return TDT_ERR_BAD_STRIDE;
  if (!aligned_to(logits, elt) || !aligned_to(dur_logits, elt)) return TDT_ERR_BAD_STRIDE;
  if (grads && (!aligned_to(grad_logits, elt) || !aligned_to(grad_dur_logits, elt))) return TDT_ERR_BAD_STRIDE;

  Params& p = *pp;
  memset(&p, 0, sizeof p);
  p.B = (int)B;
  p.Tmax = (int)T_max;
  p.U1max = (int)U1_max;
  p.V = (int)V;
  p.D = num_durations;
  p.blank = blank;
  p.red = reduction;
  p.dtype = dtype;
  p.KD = L.KD;
  p.A = L.A;
  p.Bb = L.Bb;
  p.box = L.box;
  p.triA = (int64_t)L.A * (L.A + 1) / 2;
  p.DM = L.DM;
  p.NW = L.NW;
  p.NP = L.NP;
  p.LG = L.LG;
  p.RS = L.RS;
  p.R = L.R;
  p.link = L.link;
  p.xns = L.xns;
  p.nT = L.nT;
  p.nU = L.nU;
  p.TT = L.TT;
  p.nseg = L.nseg;
  p.nch = L.nch;
  p.gnseg = L.gnseg;
  p.gnch = L.gnch;
  p.sigma = sigma;
  p.fd_nseg = tdt::make_fastdiv((uint32_t)L.nseg);
  p.fd_gnseg = tdt::make_fastdiv((uint32_t)L.gnseg);
  p.fd_u1 = tdt::make_fastdiv((uint32_t)U1_max);
  p.fd_tu1 = tdt::make_fastdiv((uint32_t)T_max * (uint32_t)U1_max);
  p.fd_a = tdt::make_fastdiv((uint32_t)L.A);
  for (int d = 0; d <= tdt::kMaxDval; ++d) p.didx[d] = -1;
  for (int i = 0; i < num_durations; ++i) {
    p.dval[i] = durations[i];
    p.didx[durations[i]] = i;
  }
  p.tok = logits;
  p.ts0 = logits_strides[0];
  p.ts1 = logits_strides[1];
  p.ts2 = logits_strides[2];
  p.dur = dur_logits;
  p.ds0 = dur_strides[0];
  p.ds1 = dur_strides[1];
  p.ds2 = dur_strides[2];
  p.labels = labels;
  p.lab_stride = labels_stride;
  p.Tlen = logit_lengths;
  p.Ulen = label_lengths;
  p.loss = loss_out;
  p.ustatus = utt_status;
  if (grads) {
    p.gtok = grad_logits;
    p.gs0 = grad_strides[0];
    p.gs1 = grad_strides[1];
    p.gs2 = grad_strides[2];
    p.gdur = grad_dur_logits;
    p.gds0 = grad_dur_strides[0];
    p.gds1 = grad_dur_strides[1];
    p.gds2 = grad_dur_strides[2];
  }
  // short rows of a batch far larger than the last-level cache are streamed past it (the
  // gradient pass re-reads little of it from there): B16 Tmax400 U1max101 V1025 fp16
  // 0.617 -> 0.596 ms per step, B2 T1000 U1500 V1025 bf16 about 1% (both with the
  // short-row gradient pass in reverse node order).  (Every long row nontemporal: B4 T200
  // U40 V8193 bf16 row pass 96 -> 83 us but gradient pass 159 -> 178 us.)
  const double row_bytes = (double)(V + num_durations) * (double)elt;
  const double padded_nodes = (double)B * (double)T_max * (double)U1_max;
  p.rows_nt = padded_nodes * row_bytes > 2.0 * tdt::kLastLevelCacheBytes ? 1 : 0;
  // long rows: every row but those of the last 224 MB (7/8 of the last-level cache) is
  // streamed past it; the gradient pass, walking the rows in reverse, starts on the ones
  // kept there (B4 T200 U40 V8193 bf16: 0.328 -> 0.307 ms per step when first measured,
  // row pass 96 -> 85 us and gradient pass 160 -> 151 us; with one row task per wave,
  // keeping 192 / 224 / 256 / 288 MB: 0.304 / 0.3003-0.3008 / 0.3027-0.3030 / 0.313 ms,
  // fp32 0.552 / 0.549 / 0.548 / 0.551 ms)
  const double keep = 0.875 * tdt::kLastLevelCacheBytes / row_bytes;
  p.nt_nodes = padded_nodes > keep ? (uint32_t)(padded_nodes - keep) : 0u;
  p.spin = 1 << 20;
  if (const char* e = getenv("TDT_LINK_SPIN_LIMIT")) {  // tests: force the waits to give up
    const long v = strtol(e, nullptr, 10);
    if (v >= 1 && v < (1 << 20)) p.spin = (int)v;
  }
  char* ws = (char*)workspace;
  p.part = (float*)(ws + L.off_part);
  p.stat = (float2*)(ws + L.off_stat);
  p.lg = (double*)(ws + L.off_lg);
  p.pw = L.pw_bytes ? (double*)(ws + L.off_pw) : nullptr;
  p.ar = ws + L.off_ar;
  p.br = ws + L.off_br;
  p.lx = ws + L.off_lx;
  p.logp = (double*)(ws + L.off_logp);
  p.wts = (double*)(ws + L.off_wts);
  p.pm = (double*)(ws + L.off_pm);
  p.pe = (int*)(ws + L.off_pe);
  p.uok = (int*)(ws + L.off_uok);
  p.xflag = (int*)(ws + L.off_xflag);
  p.xctl = L.xns ? (tdt::XCtl*)(ws + L.off_xctl) : nullptr;
  p.xprod = L.xns ? (int*)(ws + L.off_xprod) : nullptr;
  p.xring = L.xns ? ws + L.off_xring : nullptr;

  // Row and gradient chunks coincide when the logits and gradient rows share their
  // address modulo 16 bytes for every node.
  bool aligned = false;
  if (grads) {
    const int64_t e = (int64_t)elt;
    aligned = ((uintptr_t)logits % 16) == ((uintptr_t)grad_logits % 16);
    for (int d = 0; d < 3; ++d) aligned = aligned && (((logits_strides[d] - grad_strides[d]) * e) % 16 == 0);
  }
  *grads_out = grads;
  *aligned_out = aligned;
  return TDT_OK;
}

hipError_t launch_rows(const Params& p, bool aligned, hipStream_t s, int which) {
  return p.dtype == 0 ? tdt::launch_rows_f32(p, aligned, s, which)
                      : (p.dtype == 1 ? tdt::launch_rows_f16(p, aligned, s, which)
                                      : tdt::launch_rows_bf16(p, aligned, s, which));
}

int fwd_bwd_impl(int32_t dtype, int64_t B, int64_t T_max, int64_t U1_max, int64_t V, const void* logits,
                 const int64_t* logits_strides, const void* dur_logits, const int64_t* dur_strides,
                 int32_t num_durations, const int64_t* labels, int64_t labels_stride, const int64_t* logit_lengths,
                 const int64_t* label_lengths, const int32_t* durations, int32_t blank, double sigma,
                 int32_t reduction, float* loss_out, void* grad_logits, const int64_t* grad_strides,
                 void* grad_dur_logits, const int64_t* grad_dur_strides, int32_t* utt_status, void* workspace,
                 size_t workspace_bytes, void* stream, void* const* events, int32_t num_events) {
  Params p;
  bool grads = false, aligned = false;
  const int rc = prepare(dtype, B, T_max, U1_max, V, logits, logits_strides, dur_logits, dur_strides, num_durations,
                         labels, labels_stride, logit_lengths, label_lengths, durations, blank, sigma, reduction,
                         loss_out, true, false, grad_logits, grad_strides, grad_dur_logits, grad_dur_strides,
                         utt_status, workspace, workspace_bytes, &p, &grads, &aligned);
  if (rc != TDT_OK) return rc;

  hipStream_t st = (hipStream_t)stream;
  // events: 4 = {start, end, before the gradient pass, after it}; 7 = phase boundaries
  const bool phases = num_events == 7;
  auto rec = [&](int i) {
    if (events && i < num_events && events[i]) (void)hipEventRecord((hipEvent_t)events[i], st);
  };
  // with gradients, extra waves of the first lattice launch zero the padding rows of the
  // gradient while the sweeps run (only for a gradient that is one contiguous joint tensor
  // [B, Tmax, U1max, V + D]: the padding rows of a frame are then one byte range).  192
  // waves: B16 Tmax400 U1max101 V1025 fp16 (774 MB of padding rows beside the sweeps)
  // 0.603 / 0.575 / 0.546 / 0.558 / 0.556 / 0.591 ms per step with 128 / 160 / 192 / 256 /
  // 384 / 512 waves (more waves slow the sweeps, bound by the latency of their weight
  // loads, by more than the zeroing gains)
  if (grads) {
    const size_t elt = dtype == 0 ? 4 : 2;
    const int64_t* g = grad_strides;
    const int64_t* gd = grad_dur_strides;
    const bool joint = g[2] == V + num_durations && g[1] == U1_max * g[2] && g[0] == T_max * g[1] &&
                       gd[0] == g[0] && gd[1] == g[1] && gd[2] == g[2] &&
                       (const char*)grad_dur_logits == (const char*)grad_logits + V * elt;
    if (joint) p.zrows = (int)std::min<int64_t>(192, B * T_max);
  }
  rec(0);
  if (launch_rows(p, aligned, st, 0) != hipSuccess) return TDT_ERR_HIP;
  if (phases) rec(1);
  if (tdt::launch_lattice_side(p, 0, st) != hipSuccess) return TDT_ERR_HIP;
  if (phases) rec(2);
  if (tdt::launch_lattice_side(p, 1, st) != hipSuccess) return TDT_ERR_HIP;
  if (phases) rec(3);
  // coefficients (and the loss reduction) by a kernel of their own for long rows; the
  // short-row gradient pass computes them itself
  const bool coef = grads && !tdt::short_grad_rows(p, aligned);
  if (coef && tdt::launch_lattice_side(p, 2, st) != hipSuccess) return TDT_ERR_HIP;
  rec(phases ? 4 : 2);
  if (grads && launch_rows(p, aligned, st, 1) != hipSuccess) return TDT_ERR_HIP;
  rec(phases ? 5 : 3);
  // with gradients the coefficient kernel or the gradient pass has reduced the loss already
  if (!grads && tdt::launch_lattice_side(p, 3, st) != hipSuccess) return TDT_ERR_HIP;
  rec(phases ? 6 : 1);
  return TDT_OK;
}

}  // namespace

extern "C" int tdt_loss_fwd_bwd(int32_t dtype, int64_t B, int64_t T_max, int64_t U1_max, int64_t V,
                                const void* logits, const int64_t* logits_strides, const void* dur_logits,
                                const int64_t* dur_strides, int32_t num_durations, const int64_t* labels,
                                int64_t labels_stride, const int64_t* logit_lengths, const int64_t* label_lengths,
                                const int32_t* durations, int32_t blank, double sigma, int32_t reduction,
                                float* loss_out, void* grad_logits, const int64_t* grad_strides,
                                void* grad_dur_logits, const int64_t* grad_dur_strides, int32_t* utt_status,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_bwd_impl(dtype, B, T_max, U1_max, V, logits, logits_strides, dur_logits, dur_strides, num_durations,
                      labels, labels_stride, logit_lengths, label_lengths, durations, blank, sigma, reduction,
                      loss_out, grad_logits, grad_strides, grad_dur_logits, grad_dur_strides, utt_status, workspace,
                      workspace_bytes, stream, nullptr, 0);
}

extern "C" int tdt_loss_fwd_bwd_timed(int32_t dtype, int64_t B, int64_t T_max, int64_t U1_max, int64_t V,
                                      const void* logits, const int64_t* logits_strides, const void* dur_logits,
                                      const int64_t* dur_strides, int32_t num_durations, const int64_t* labels,
                                      int64_t labels_stride, const int64_t* logit_lengths,
                                      const int64_t* label_lengths, const int32_t* durations, int32_t blank,
                                      double sigma, int32_t reduction, float* loss_out, void* grad_logits,
                                      const int64_t* grad_strides, void* grad_dur_logits,
                                      const int64_t* grad_dur_strides, int32_t* utt_status, void* workspace,
                                      size_t workspace_bytes, void* stream, void* const* events,
                                      int32_t num_events) {
  if (!events || (num_events != 4 && num_events != 7)) return TDT_ERR_INVALID_ARGUMENT;
  return fwd_bwd_impl(dtype, B, T_max, U1_max, V, logits, logits_strides, dur_logits, dur_strides, num_durations,
                      labels, labels_stride, logit_lengths, label_lengths, durations, blank, sigma, reduction,
                      loss_out, grad_logits, grad_strides, grad_dur_logits, grad_dur_strides, utt_status, workspace,
                      workspace_bytes, stream, events, num_events);
}

extern "C" int tdt_loss_backward(int32_t dtype, int64_t B, int64_t T_max, int64_t U1_max, int64_t V,
                                 const void* logits, const int64_t* logits_strides, const void* dur_logits,
                                 const int64_t* dur_strides, int32_t num_durations, const int64_t* labels,
                                 int64_t labels_stride, const int64_t* logit_lengths, const int64_t* label_lengths,
                                 const int32_t* durations, int32_t blank, double sigma, int32_t reduction,
                                 const float* grad_loss, void* grad_logits, const int64_t* grad_strides,
                                 void* grad_dur_logits, const int64_t* grad_dur_strides, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  Params p;
  bool grads = false, aligned = false;
  const int rc = prepare(dtype, B, T_max, U1_max, V, logits, logits_strides, dur_logits, dur_strides, num_durations,
                         labels, labels_stride, logit_lengths, label_lengths, durations, blank, sigma, reduction,
                         nullptr, false, true, grad_logits, grad_strides, grad_dur_logits, grad_dur_strides,
                         nullptr, workspace, workspace_bytes, &p, &grads, &aligned);
  if (rc != TDT_OK) return rc;
  p.gscale = grad_loss;
  hipStream_t st = (hipStream_t)stream;
  if (!tdt::short_grad_rows(p, aligned) && tdt::launch_lattice_side(p, 2, st) != hipSuccess) return TDT_ERR_HIP;
  if (launch_rows(p, aligned, st, 1) != hipSuccess) return TDT_ERR_HIP;
  return TDT_OK;
}

// ------------------------------------------------------------------------------------
// Allocation-free entry point.  The workspace lives in a file-scope device array (one
// copy per GPU, held until the process ends).  In host code `scratch` names a host-side
// stand-in, never a device address: the address of each GPU's copy is taken once per
// device with hipGetSymbolAddress (with that device current) and only that address is
// passed to the kernels.
static_assert(TDT_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte blocks");
static __device__ __align__(256) unsigned char scratch[TDT_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this GPU's scratch copy for work on `stream` (the stream's
// device; the current device for the null stream), or NULL on a HIP error.
void* scratch_for(hipStream_t stream) {
  int dev = -1;
  if (stream) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int tdt_loss_fwd_bwd_noalloc(int32_t dtype, int64_t B, int64_t T_max, int64_t U1_max, int64_t V,
                                        const void* logits, const int64_t* logits_strides, const void* dur_logits,
                                        const int64_t* dur_strides, int32_t num_durations, const int64_t* labels,
                                        int64_t labels_stride, const int64_t* logit_lengths,
                                        const int64_t* label_lengths, const int32_t* durations, int32_t blank,
                                        double sigma, int32_t reduction, float* loss_out, void* grad_logits,
                                        const int64_t* grad_strides, void* grad_dur_logits,
                                        const int64_t* grad_dur_strides, int32_t* utt_status, void* stream) {
  // every host check first (against a placeholder workspace address that is validated
  // but never used), so that invalid arguments and oversized calls touch no HIP state
  {
    Params p;
    bool grads = false, aligned = false;
    void* const placeholder = (void*)(uintptr_t)256;
    const int rc = prepare(dtype, B, T_max, U1_max, V, logits, logits_strides, dur_logits, dur_strides,
                           num_durations, labels, labels_stride, logit_lengths, label_lengths, durations, blank,
                           sigma, reduction, loss_out, true, false, grad_logits, grad_strides, grad_dur_logits,
                           grad_dur_strides, utt_status, placeholder, (size_t)TDT_NOALLOC_SCRATCH_BYTES, &p, &grads,
                           &aligned);
    if (rc != TDT_OK) return rc;
  }
  void* ws = scratch_for((hipStream_t)stream);
  if (!ws) return TDT_ERR_HIP;
  return fwd_bwd_impl(dtype, B, T_max, U1_max, V, logits, logits_strides, dur_logits, dur_strides, num_durations,
                      labels, labels_stride, logit_lengths, label_lengths, durations, blank, sigma, reduction,
                      loss_out, grad_logits, grad_strides, grad_dur_logits, grad_dur_strides, utt_status, ws,
                      (size_t)TDT_NOALLOC_SCRATCH_BYTES, stream, nullptr, 0);
}
