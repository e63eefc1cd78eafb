// nha_internal.h -- host-side plumbing shared by the C ABI and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/nha.h"

namespace nha {

// RoPE frequencies theta_i = base^(-2i/d), computed on the host in double,
// and the position of row 0 of the sequence (0, or where a continued segment
// starts): row t is rotated by (pos0 + t) theta_i.
struct RopeTheta {
  double theta[64];
  long long pos0;
};

// Problem shape after validation.
struct Shape {
  int B, T, H, Hkv, d, m, w, C;
  int sh;     // absorption shift: token t - sh enters the slots at step t >= sh (w, or 0 without token shift)
  int G;      // H / Hkv
  int mp;     // m padded to a multiple of 32
  int NC;     // ceil(T / C)
  int NQ;     // ceil(T / 64) query tiles of the window kernels
  bool rope;  // RoPE enabled
  bool win;   // w > 0
  float scale;
  int dtype;
  int esz;    // element bytes
};

// The forward runs both branches in one chunk kernel (bf16 inputs, C = 64:
// a 128-query window tile is two chunks) when the slot-state scan has at
// least 256 waves (one per batch row, KV head and 16 state columns): the scan
// walks the chunks in order, and with fewer waves the chip is mostly idle
// while it runs, so a separate window kernel, which needs no states and runs
// beside the scan on the side stream, does better.  Otherwise a window kernel
// and a slot kernel joined through the window partial in the workspace.
inline bool chunk_fused(const Shape& s) {
  return s.esz == 2 && s.C == 64 && (long long)s.B * s.Hkv * (s.d / 16) >= 256;
}

// Segments of the bf16 slot-state scan.  The scan walks the chunks in order
// with one single-wave workgroup per (batch row, KV head, 16 state columns);
// below 256 such waves most of the chip idles through that walk, and on
// walks of 384 chunks or more the chunks are cut into n segments of len
// chunks (up to 768 waves in all, at least 8 chunks a segment): every
// segment's end state from a zero start, then the segments' start states in
// order, then every segment walked again from its start state, writing the
// chunk-start states.  On shorter walks the single walk runs beside the
// window branch, which the segments' extra waves would crowd out.
struct ScanSegs {
  int n, len;
};
inline ScanSegs scan_segments(const Shape& s) {
  ScanSegs r{1, s.NC};
  if (s.esz != 2 || s.m == 0) return r;
  const long long base = (long long)s.B * s.Hkv * (s.d / 16);
  if (base >= 256 || s.NC < 384) return r;
  int n = (int)(768 / base);
  if (n > 16) n = 16;
  if (n > s.NC / 8) n = s.NC / 8;
  if (n < 2) return r;
  r.len = (s.NC + n - 1) / n;
  r.n = (s.NC + r.len - 1) / r.len;  // no empty segment
  return r;
}

// dalpha's cross-chunk carry (bf16 inputs): exact at every kCarryStride-th
// chunk, summed from chunk totals in between.
constexpr int kCarryStride = 16;
inline int carry_ckpts(const Shape& s) { return s.esz == 2 && s.m > 0 ? (s.NC - 1) / kCarryStride : 0; }

constexpr size_t kMaxLds = 160 * 1024;  // LDS bytes per workgroup on gfx950

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Forward workspace carve-up (offsets in bytes from the workspace base).
struct FwdWs {
  size_t sst;    // chunk-start states: [B*Hkv][NC][ SK | SV ], each mp x d (dtype): fp32 as
                 // [i][d] rows, bf16 in column blocks [d/16][i][16]
  size_t wt;     // per-chunk absorption weights W^T: [B*Hkv][NC][mp][C]       (dtype)
  size_t aend;   // per-chunk decay exp(G_end): [B*Hkv][NC][mp]                (float)
  size_t seg;    // segmented scan: end / start states [2][B*Hkv*n][m][d], decays [B*Hkv*n][mp] (float)
  size_t qrot;   // RoPE'd q: [B][T][H][d]                                       (dtype)
  size_t krot;   // RoPE'd k: [B][T][Hkv][d]                                     (dtype)
  size_t rcs;    // RoPE angles (cos, sin)(t theta_i): [T][d/2]                   (float2)
  size_t ol;     // slot-branch partial output o_L / Z_L: [B][T][H][d]          (dtype)
  size_t lsel;   // slot-branch partial lse: [B][H][T]                           (float)
  size_t total;
};

inline FwdWs fwd_ws_layout(const Shape& s) {
  FwdWs L;
  size_t off = 0;
  size_t units = (size_t)s.B * s.Hkv;
  L.sst = off;
  off += align256(units * s.NC * 2 * (size_t)s.mp * s.d * s.esz);
  L.wt = off;
  off += align256(units * s.NC * (size_t)s.mp * s.C * s.esz);
  L.aend = off;
  off += align256(units * s.NC * (size_t)s.mp * 4);
  L.seg = off;
  {
    const ScanSegs sg = scan_segments(s);
    if (sg.n > 1) off += align256(units * sg.n * (2 * (size_t)s.m * s.d + s.mp) * 4);
  }
  L.qrot = off;
  if (s.rope && s.win) off += align256((size_t)s.B * s.T * s.H * s.d * s.esz);
  L.krot = off;
  if (s.rope && s.win) off += align256((size_t)s.B * s.T * s.Hkv * s.d * s.esz);
  L.rcs = off;
  if (s.rope && s.win) off += align256((size_t)s.T * (s.d / 2) * 8);
  L.ol = off;
  off += align256((size_t)s.B * s.T * s.H * s.d * s.esz);
  L.lsel = off;
  off += align256((size_t)s.B * s.H * s.T * 4);
  L.total = off;
  return L;
}

// Decode-state carve-up (see nha_decode_state_size in nha.h).
// The decode step splits each (batch, KV head)'s keys over up to
// kDecodeSplitMax workgroups; their partial softmax results are combined by a
// second launch through the `part` region of the state.
constexpr int kDecodeSplitMax = 32;
struct StateLayout {
  size_t sk, sv, rk, rv, rkr, pos, part, total;
};
inline StateLayout state_layout(const Shape& s) {
  StateLayout L;
  size_t units = (size_t)s.B * s.Hkv, off = 0;
  L.sk = off;
  off += align256(units * s.m * s.d * 4);
  L.sv = off;
  off += align256(units * s.m * s.d * 4);
  L.rk = off;
  off += align256(units * (size_t)s.w * s.d * s.esz);
  L.rv = off;
  off += align256(units * (size_t)s.w * s.d * s.esz);
  L.rkr = off;  // RoPE'd keys of the ring (only with RoPE)
  off += align256(s.rope ? units * (size_t)s.w * s.d * s.esz : 0);
  L.pos = off;
  off += align256(units * 8);
  L.part = off;  // [B*H][kDecodeSplitMax][d + 4] float: max, sum, -, -, o
  off += align256((size_t)s.B * s.H * kDecodeSplitMax * (s.d + 4) * 4);
  L.total = off;
  return L;
}
// Workgroups per (batch, KV head) of a decode step: enough to fill the chip,
// at least 8 keys each, at most kDecodeKeysPerSplit (so m + w <=
// kDecodeSplitMax * kDecodeKeysPerSplit, checked by the API).  `small`: every
// split has at most kDecodeKeysPerSplit / 2 keys, so the half-size key groups
// serve it.
constexpr int kDecodeKeysPerSplit = 128;
struct DecodeSplit {
  int ns;
  bool small;
};
inline DecodeSplit decode_splits(const Shape& s) {
  const int units = s.B * s.Hkv, keys = s.m + s.w;
  int ns = 256 / (units > 0 ? units : 1);
  if (ns > kDecodeSplitMax) ns = kDecodeSplitMax;
  if (ns > keys / 8) ns = keys / 8;
  const int half = kDecodeKeysPerSplit / 2;
  const int need_small = (keys + half - 1) / half;
  if (need_small <= kDecodeSplitMax) {
    if (ns < need_small) ns = need_small;
    return {ns < 1 ? 1 : ns, true};
  }
  const int need = (keys + kDecodeKeysPerSplit - 1) / kDecodeKeysPerSplit;
  if (ns < need) ns = need;
  return {ns < 1 ? 1 : ns, false};
}

// A second stream for the launches of one call that do not depend on each
// other (RoPE beside the gate products and the state scan; the window dq
// beside the adjoint scan; the dalpha carry beside the window dk/dv).  The
// side stream is created once per thread and device (default priority,
// non-blocking) with two events; every call joins its side-stream work back
// into the caller's stream before it returns, so the caller sees one stream.
// `side` is null -- everything runs on the caller's stream, in order -- for
// the timed calls (their per-launch events measure one kernel each) and when
// the stream cannot be created.
struct Fork {
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr, ev_mid = nullptr;
  // fork point: the side stream's next launches start after everything
  // enqueued on `main` so far (launches enqueued on `main` after this point
  // are not waited for)
  void record(hipStream_t main) const {
    if (side) (void)hipEventRecord(ev_fork, main);
  }
  // the stream for launches that follow the last fork point
  hipStream_t follow(hipStream_t main) const {
    if (!side) return main;
    (void)hipStreamWaitEvent(side, ev_fork, 0);
    return side;
  }
  hipStream_t begin(hipStream_t main) const {
    record(main);
    return follow(main);
  }
  // a later point on `main` (mark_mid) that the side stream's following
  // launches wait for (wait_mid), without a new fork
  void mark_mid(hipStream_t main) const {
    if (side) (void)hipEventRecord(ev_mid, main);
  }
  void wait_mid() const {
    if (side) (void)hipStreamWaitEvent(side, ev_mid, 0);
  }
  // `main` continues after everything enqueued on the side stream so far
  void join(hipStream_t main) const {
    if (!side) return;
    (void)hipEventRecord(ev_join, side);
    (void)hipStreamWaitEvent(main, ev_join, 0);
  }
};
Fork side_fork(bool enabled);

// Records caller-provided timing events around consecutive launches.
struct Marks {
  void* const* ev = nullptr;
  int i = 0;
  void mark(hipStream_t st) {
    if (ev) (void)hipEventRecord((hipEvent_t)ev[i], st);
    ++i;
  }
};

// Launch sequence of one forward / backward call (names are static strings).
int fwd_stages(const Shape& s, bool with_state, const char** names, int max);
int bwd_stages(const Shape& s, bool after_fwd, const char** names, int max);

// ---------------------------------------------------------------- launchers
// Shared first stages of the forward and the backward: RoPE of q and k (when
// enabled and w > 0), per-chunk gate products, and the scan that writes the
// slot state at every chunk start (and optionally the final fp32 state).
struct ProloguePtrs {
  void* sst;
  void* wt;
  float* aend;
  void* qrot;  // nullable when RoPE is off or w == 0
  void* krot;
  float2* rcs;  // RoPE (cos, sin) table, same condition
  float* skout;  // nullable
  float* svout;
  const float* s0k = nullptr;  // initial slot states [B*Hkv][m][d], nullable = zero
  const float* s0v = nullptr;
  float* seg = nullptr;  // the segmented scan's state rows (scan_segments n > 1)
};
hipError_t launch_prologue(const Shape& s, const RopeTheta& th, const void* q, const void* k, const void* v,
                           const void* alpha, const ProloguePtrs& pp, Marks& mk, hipStream_t st, const Fork& fk);

// Compute units of the current device (cached per device); persistent
// kernels size their grids with it.
int device_cu_count();

// Each returns hipSuccess or the launch error.  All launches go on `st`.
struct FwdPtrs {
  const void *q, *k, *v, *alpha;
  void* o;
  float* lse;
  void* state_out;  // nullable
  char* ws;
  void* const* events;  // nullable timing events
  const float* s0k = nullptr;  // initial slot states [B*Hkv][m][d], nullable = zero
  const float* s0v = nullptr;
  bool one_stream = false;      // every launch on the caller's stream (no side stream)
  // weighted-fusion ablation: the window branch starts from an empty softmax
  // (its own) instead of the slot partial and writes its own normalised read
  // to o and its lse to lse; the slot partial o_L / Z_L and its lse go to
  // ol_dst / lsel_dst (null: the workspace)
  bool separate = false;
  void* ol_dst = nullptr;
  float* lsel_dst = nullptr;
};
hipError_t launch_fwd(const Shape& s, const RopeTheta& th, const FwdPtrs& p, hipStream_t st);

struct DecodePtrs {
  const void *q, *k, *v, *alpha;
  void* state;
  void* o;
};
hipError_t launch_decode(const Shape& s, const RopeTheta& th, const DecodePtrs& p, hipStream_t st);

size_t bwd_ws_bytes(const Shape& s);
struct BwdPtrs {
  const void *q, *k, *v, *alpha, *o, *dO;
  const float* lse;
  void *dq, *dk, *dv;
  float* dalpha;
  char* ws;
  void* const* events;  // nullable timing events
  bool after_fwd;       // the workspace already holds this input's forward prologue
  const float* s0k = nullptr;  // initial slot states [B*Hkv][m][d], nullable = zero
  const float* s0v = nullptr;
  float* ds0k = nullptr;  // their gradients, nullable
  float* ds0v = nullptr;
  // weighted-fusion ablation: the window kernels' own dO, lse and D_t (null:
  // the slot kernels' dO, lse and D_t, i.e. the unified softmax)
  const void* win_dO = nullptr;
  const float* win_lse = nullptr;
  const float* win_D = nullptr;
};
hipError_t launch_bwd(const Shape& s, const RopeTheta& th, const BwdPtrs& p, hipStream_t st);

// The device address of the allocation-free forward's scratch array on the
// current device (looked up once per device with hipGetSymbolAddress) and its
// size in bytes.
constexpr size_t kNoallocScratchBytes = NHA_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void** ptr);

// Weighted-fusion ablation (separate slot and window softmaxes mixed by a
// per-(token, head) coefficient lam [B][T][H] fp32).
size_t weighted_ws_bytes(const Shape& s);
struct WeightedPtrs {
  const void *q, *k, *v, *alpha;
  const float* lam;
  void* o;       // forward output (nullable in the backward)
  float* lse2;   // forward: nullable [2][B][H][T] (slot lse, window lse)
  const void* dO;  // backward
  void *dq, *dk, *dv;
  float* dalpha;
  float* dlam;   // nullable
  char* ws;
};
hipError_t launch_fwd_weighted(const Shape& s, const RopeTheta& th, const WeightedPtrs& p, hipStream_t st);
hipError_t launch_bwd_weighted(const Shape& s, const RopeTheta& th, const WeightedPtrs& p, hipStream_t st);

// Chunked prefill: a segment continuing a decode state.  s is the segment's
// shape, se the extended shape (T + P rows: the P = min(pos0, w) ring tokens
// first); th.pos0 = pos0 - P, the absolute position of extended row 0.
struct ContPtrs {
  const void *q, *k, *v, *alpha;
  const void* state_in;
  void* o;          // forward: output; backward: the forward's output (read)
  float* lse;       // forward: nullable output; backward: the forward's lse (read)
  void* state_out;  // forward, nullable
  const void* dO;
  void *dq, *dk, *dv;
  float* dalpha;
  float *ds0k, *ds0v;  // gradients of the state's slots, [B][Hkv][m][d]
  void *drk, *drv;     // gradients of the state's ring keys / values, ring layout, nullable
  char* ws;
};
size_t cont_ws_bytes(const Shape& se, bool bwd);
hipError_t launch_fwd_continue(const Shape& s, const Shape& se, const RopeTheta& th, const ContPtrs& p,
                               hipStream_t st);
hipError_t launch_bwd_continue(const Shape& s, const Shape& se, const RopeTheta& th, const ContPtrs& p,
                               hipStream_t st);

// LDS bytes the largest forward / backward kernel needs for this shape.
size_t slot_fwd_lds_bytes(const Shape& s);
size_t slot_bwd_lds_bytes(const Shape& s);

}  // namespace nha
