// C ABI of one TSP rank's layer share (declared in include/tsp.h): argument
// validation, workspace carving and the double-buffered shard stream.
//
// Shard stream.  The TSP schedules (section 2 of "Folding Tensor and Sequence
// Parallelism for Memory-Efficient Transformer Training & Inference") move
// weight shards between ranks: a broadcast per attention iteration, a ring
// step per MLP shard, and an all-gather of K/V along the sequence; the
// transfers are pipelined behind the GEMMs.  Here the other ranks' shards are
// device buffers, and the transfer becomes a copy into one of two workspace
// slots on a side stream.  Events hand each slot over:
//   copy stream:    wait free[s] (slot s released by iteration i-2) -> copy -> record ready[s]
//   compute stream: wait ready[s] -> GEMM / attention / GEMM -> record free[s]
// so the copy of iteration i+1 runs while iteration i computes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "tsp.h"
#include "tsp_kernels.h"

using namespace tsp;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIP_TRY(expr)                                                                       \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ != hipSuccess)                                                                   \
      return fail(TSP_E_HIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_), __FILE__, \
                  __LINE__);                                                                \
  } while (0)

// S, C and T are per sequence; the micro-batch holds B sequences, so the
// rank has BT = B*T local rows and the gathered K/V BS = B*S positions per head.
// Hkv K/V heads, Hkd = Hkv/D of them per shard, ks = Hkd*d K (V) rows per
// shard; rope_theta = 0 means no rotary embedding.
struct Dims {
  int64_t h, H, d, F, D, r, S, C, T, Hd, hs, Fs, B, BT, BS, Hkv, Hkd, ks;
  size_t es;
  Dtype dt;
  float eps;
  float rope_theta;
  uint32_t flags;
};

int64_t acc_group(const Dims& d);

// The GEMM and attention kernels stage operands through buffer loads whose
// byte offsets are 32-bit and which mark rows and chunks outside a matrix
// with the offset 2^31 (past the range, so they read zero).  Every buffer
// range they address must therefore stay at or below 2^31 bytes; larger
// shapes are refused before anything is enqueued.
constexpr uint64_t kMaxRange = 1ull << 31;

int check_offsets(const Dims& d) {
  const int64_t G = acc_group(d);
  const uint64_t es = d.es, BT = d.BT, h = d.h;
  // GEMM A operands, [B*T rows][K]: the normalised activations (K = h), an
  // accumulation group's attention outputs (G*hs) or SwiGLU products (G*Fs),
  // and in the MLP backward [da | db] (2*Fs) and its transpose.
  const uint64_t widest = std::max<uint64_t>({(uint64_t)h, (uint64_t)(G * d.hs), (uint64_t)(G * d.Fs),
                                              (uint64_t)(2 * d.Fs)});
  const uint64_t a_op = BT * widest * es;
  // GEMM B operands: the packed Q|K|V block, the W_O and W2 group buffers,
  // the W1|W3 block and its transpose.
  const uint64_t b_op = std::max<uint64_t>({(uint64_t)(d.hs + 2 * d.ks) * h, h * (uint64_t)(G * d.hs),
                                            h * (uint64_t)(G * d.Fs), 2 * (uint64_t)d.Fs * h}) * es;
  // Attention: one sequence's K plane of a K/V head, and the V^T plane of a
  // K/V head over the micro-batch ((d-1) rows of B*S keys, then S).
  const uint64_t k_plane = (uint64_t)d.S * d.d * es;
  const uint64_t v_plane = ((uint64_t)(d.d - 1) * d.BS + d.S) * es;
  struct {
    const char* what;
    uint64_t bytes;
  } rs[] = {{"an activation GEMM operand", a_op}, {"a weight GEMM operand", b_op},
            {"a K plane", k_plane}, {"a V^T plane", v_plane}};
  for (auto& r : rs)
    if (r.bytes > kMaxRange)
      return fail(TSP_E_SHAPE, "%s would span %llu bytes; the kernels address at most 2^31 bytes per buffer",
                  r.what, (unsigned long long)r.bytes);
  return TSP_OK;
}

int check_dims(const tsp_dims* p, Dims* o) {
  if (!p) return fail(TSP_E_INVAL, "dims is NULL");
  if (p->dtype != TSP_BF16 && p->dtype != TSP_F32)
    return fail(TSP_E_DTYPE, "dtype %d is neither TSP_BF16 nor TSP_F32", p->dtype);
  if (p->fold <= 0 || p->rank < 0 || p->rank >= p->fold)
    return fail(TSP_E_INVAL, "rank %d outside [0, fold=%d)", p->rank, p->fold);
  if (p->seq < 0 || p->hidden <= 0 || p->n_heads <= 0 || p->head_dim <= 0 || p->ffn <= 0)
    return fail(TSP_E_INVAL, "sizes must be positive (seq may be 0)");
  if (!(p->eps >= 0.f) || !std::isfinite(p->eps)) return fail(TSP_E_INVAL, "eps must be finite >= 0");
  if ((int64_t)p->n_heads * p->head_dim != p->hidden)
    return fail(TSP_E_SHAPE, "hidden %d != n_heads %d * head_dim %d", p->hidden, p->n_heads,
                p->head_dim);
  if (p->head_dim != 16 && p->head_dim != 32 && p->head_dim != 64 && p->head_dim != 128)
    return fail(TSP_E_SHAPE, "head_dim %d not in {16, 32, 64, 128}", p->head_dim);
  if (p->n_heads % p->fold) return fail(TSP_E_SHAPE, "n_heads %d %% fold %d != 0", p->n_heads, p->fold);
  if (p->ffn % p->fold) return fail(TSP_E_SHAPE, "ffn %d %% fold %d != 0", p->ffn, p->fold);
  if (p->seq % (2 * (int64_t)p->fold))
    return fail(TSP_E_SHAPE, "seq %lld is not a multiple of 2*fold", (long long)p->seq);
  if (p->seq % 8) return fail(TSP_E_SHAPE, "seq %lld is not a multiple of 8", (long long)p->seq);
  if (p->hidden % 8) return fail(TSP_E_SHAPE, "hidden %d is not a multiple of 8", p->hidden);
  if (p->batch < 0) return fail(TSP_E_INVAL, "batch %d is negative", p->batch);
  if ((int64_t)std::max(p->batch, 1) * p->seq > INT32_MAX)
    return fail(TSP_E_SHAPE, "batch * seq exceeds 2^31 - 1 positions");
  if (p->n_kv_heads < 0) return fail(TSP_E_INVAL, "n_kv_heads %d is negative", p->n_kv_heads);
  const int32_t hkv = p->n_kv_heads ? p->n_kv_heads : p->n_heads;
  if (p->n_heads % hkv)
    return fail(TSP_E_SHAPE, "n_heads %d %% n_kv_heads %d != 0", p->n_heads, hkv);
  if (hkv % p->fold) return fail(TSP_E_SHAPE, "n_kv_heads %d %% fold %d != 0", hkv, p->fold);
  if (!(p->rope_theta >= 0.f) || !std::isfinite(p->rope_theta) ||
      (p->rope_theta > 0.f && p->rope_theta <= 1.f))
    return fail(TSP_E_INVAL, "rope_theta must be 0 or a finite value > 1");
  o->h = p->hidden;
  o->H = p->n_heads;
  o->d = p->head_dim;
  o->F = p->ffn;
  o->D = p->fold;
  o->r = p->rank;
  o->S = p->seq;
  o->C = p->seq / (2 * p->fold);
  o->T = 2 * o->C;
  o->Hd = o->H / o->D;
  o->hs = o->h / o->D;
  o->Fs = o->F / o->D;
  o->Hkv = hkv;
  o->Hkd = hkv / o->D;
  o->ks = o->Hkd * o->d;
  o->rope_theta = p->rope_theta;
  o->B = std::max(p->batch, 1);
  o->BT = o->B * o->T;
  o->BS = o->B * o->S;
  o->dt = p->dtype == TSP_BF16 ? BF16 : F32;
  o->es = p->dtype == TSP_BF16 ? 2 : 4;
  o->eps = p->eps;
  o->flags = p->flags;
  return check_offsets(*o);
}

size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace regions.  Offsets are from the workspace base.
struct AttnWs {
  size_t xn, y, q, o, slotw[2], slotkv[2], bo[2], op, ml, end;
};
struct MlpWs {
  size_t xn, y, gg, slotw[2], bw[2], end;
};

// Q | K | V rows of a packed attention shard, then W_O (h rows of hs).
size_t qkv_rows(const Dims& d) { return (size_t)(d.hs + 2 * d.ks); }
size_t attn_shard_elems(const Dims& d) { return (qkv_rows(d) + d.hs) * d.h; }
size_t mlp_shard_elems(const Dims& d) { return 3 * (size_t)d.Fs * d.h; }

// Launch groups: the QKV and attention launches of a forward half each cover
// min(4, D/2) consecutive shards (one with TSP_F_SHARD_LAUNCH); the W1/W3
// launch covers two such groups when they share an accumulation group.
#ifndef TSP_ACC_GROUP
#define TSP_ACC_GROUP 4
#endif
#ifndef TSP_W13_PAIR
#define TSP_W13_PAIR 1  // W1/W3 of two launch groups in one launch (mlp_body)
#endif
int64_t launch_group(const Dims& d) {
  return std::max<int64_t>(1, std::min<int64_t>(TSP_ACC_GROUP, d.D / 2));
}

// Accumulation groups.  The O projections (and W2 projections) of G
// consecutive shards run as one GEMM with K = G*hs (G*Fs): the shards'
// attention outputs (SwiGLU products) sit side by side, and each shard's W_O
// (W2) block is copied next to the others' on the side stream.  By default
// G = D: one O and one W2 projection per layer, K = h (F), which add the
// residual in their epilogue, so no fp32 partial sum is written or read.  The
// group buffers then hold all of W_O (W2), as many bytes as two half-layer
// buffers.  With TSP_F_SHARD_LAUNCH, or when the layer's SwiGLU products
// ([B*T][F]) would outgrow the kernels' 2^31-byte operand range, G =
// min(4, D/2) (at most half of W_O or W2 held at once, D/G passes over an
// fp32 accumulator).
int64_t acc_group(const Dims& d) {
  if (d.flags & TSP_F_SHARD_LAUNCH) return launch_group(d);
  const uint64_t widest = (uint64_t)d.BT * (uint64_t)std::max<int64_t>(d.h, d.D * d.Fs) * d.es;
  return widest <= (1ull << 31) ? d.D : launch_group(d);
}
size_t kv_block_elems(const Dims& d) { return 2 * (size_t)d.Hkd * d.BS * d.d; }
size_t kv_v_offset(const Dims& d) { return (size_t)d.Hkd * d.BS * d.d; }  // elements before Vt_j

// The B sequences' items run side by side like extra heads.
AttnPlan plan_of(const Dims& d) {
  return attn_plan(d.T, d.S, d.C, (int)d.r, (int)d.D, (int)(d.Hd * d.B), attn_wide(d.dt, (int)d.d));
}

// Shards per launch in the forward halves: the P shards of a launch group
// share each QKV, attention and W1/W3 launch (TSP_F_SHARD_LAUNCH: one).  Wider launches fill the CUs with larger GEMM
// tiles and give attention more heads per launch (fewer split items); the
// two weight slots then hold 2G shards' Q|K|V (W1|W3) blocks, all of them at
// D = 8, a few hundred MB at the 7B shape.
int64_t launch_shards(const Dims& d) {
  if (d.flags & TSP_F_SHARD_LAUNCH) return 1;
  return launch_group(d);
}

// Attention plan of a launch over np shards' heads.
AttnPlan plan_for(const Dims& d, int64_t np) {
  return attn_plan(d.T, d.S, d.C, (int)d.r, (int)d.D, (int)(np * d.Hd * d.B), attn_wide(d.dt, (int)d.d));
}

// Split-partial rows a launch over np shards needs.
size_t split_rows(const Dims& d, int64_t np) {
  const AttnPlan p = plan_for(d, np);
  return p.split ? (size_t)(np * d.Hd * d.B) * p.nqt * p.maxseg * p.bq : 0;
}

AttnWs attn_ws(const Dims& d, size_t base) {
  AttnWs w;
  size_t o = base;
  const size_t act = al((size_t)d.BT * d.h * d.es);
  w.xn = o; o += act;
  const int64_t G = acc_group(d), P = launch_shards(d);
  const int ngroups = d.D > G ? 2 : 1;  // group buffers in use (double-buffered across groups)
  w.y = o;
  if (ngroups > 1) o += al((size_t)d.BT * d.h * 4);  // fp32 partial sum across groups
  w.q = o; o += al((size_t)P * d.BT * d.hs * d.es);  // [P*Hd][B*T][d]
  w.o = o; o += al((size_t)d.BT * G * d.hs * d.es);  // [B*T][G*hs]
  for (int s = 0; s < 2; s++) { w.slotw[s] = o; o += al((size_t)P * qkv_rows(d) * d.h * d.es); }
  for (int s = 0; s < 2; s++) { w.slotkv[s] = o; o += al((size_t)P * kv_block_elems(d) * d.es); }
  for (int s = 0; s < 2; s++) {  // [h][G*hs]
    w.bo[s] = o;
    if (s < ngroups) o += al((size_t)d.h * G * d.hs * d.es);
  }
  size_t nslot = split_rows(d, P);
  if (d.D % P) nslot = std::max(nslot, split_rows(d, d.D % P));  // the last, shorter launch
  w.op = o; o += al(nslot * d.d * 4);
  w.ml = o; o += al(nslot * 2 * 4);
  w.end = o;
  return w;
}

MlpWs mlp_ws(const Dims& d, size_t base) {
  MlpWs w;
  size_t o = base;
  const int64_t G = acc_group(d), P = launch_shards(d);
  const int ngroups = d.D > G ? 2 : 1;
  w.xn = o; o += al((size_t)d.BT * d.h * d.es);
  w.y = o;
  if (ngroups > 1) o += al((size_t)d.BT * d.h * 4);
  w.gg = o; o += al((size_t)d.BT * G * d.Fs * d.es);  // [B*T][G*Fs]
  // [W1 of the launch's shards | their W3]
  for (int s = 0; s < 2; s++) { w.slotw[s] = o; o += al(2 * (size_t)P * d.Fs * d.h * d.es); }
  for (int s = 0; s < 2; s++) {  // [h][G*Fs]
    w.bw[s] = o;
    if (s < ngroups) o += al((size_t)d.h * G * d.Fs * d.es);
  }
  w.end = o;
  return w;
}

size_t kv_ws_bytes(const Dims& d) { return al((size_t)d.BT * d.h * d.es); }

bool aligned(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Events for the slot hand-offs, created once per host thread and device.
struct Events {
  hipEvent_t start, join, readyA[2], freeA[2], readyM[2], freeM[2], freeO[2], freeW[2];
};
constexpr int kMaxDev = 64;
// One host thread's events for each device, destroyed when the thread ends.
struct EventSets {
  Events* ev[kMaxDev] = {};
  ~EventSets() {
    for (Events* e : ev) {
      if (!e) continue;
      hipEvent_t* all[] = {&e->start,    &e->join,     &e->readyA[0], &e->readyA[1],
                           &e->freeA[0], &e->freeA[1], &e->readyM[0], &e->readyM[1],
                           &e->freeM[0], &e->freeM[1], &e->freeO[0],  &e->freeO[1],
                           &e->freeW[0], &e->freeW[1]};
      for (hipEvent_t* p : all)
        if (*p) (void)hipEventDestroy(*p);
      delete e;
    }
  }
};
thread_local EventSets g_events;
thread_local Events** const g_ev = g_events.ev;

int get_events(Events** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDev) return fail(TSP_E_HIP, "device index %d unsupported", dev);
  if (!g_ev[dev]) {
    Events* e = new Events();  // value-initialised: null handles until created
    hipEvent_t* all[] = {&e->start,    &e->join,     &e->readyA[0], &e->readyA[1],
                         &e->freeA[0], &e->freeA[1], &e->readyM[0], &e->readyM[1],
                         &e->freeM[0], &e->freeM[1], &e->freeO[0],  &e->freeO[1],
                         &e->freeW[0], &e->freeW[1]};
    for (hipEvent_t* p : all) HIP_TRY(hipEventCreateWithFlags(p, hipEventDisableTiming));
    g_ev[dev] = e;
  }
  *out = g_ev[dev];
  return TSP_OK;
}

// One call's streams: `cs` carries the copies (== s when not overlapping).
struct Ctx {
  const Dims* d;
  char* ws;
  hipStream_t s, cs;
  bool side;
  Events* ev;
  bool prof;
};

// Per-kernel timing (TSP_F_PROFILE): timing-enabled events bracket each
// launch on the compute stream; tsp_profile_read resolves them later.
struct ProfState {
  struct Pending {
    int k;
    hipEvent_t a, b;
  };
  std::vector<hipEvent_t> pool;
  std::vector<Pending> pending;
  double ms[TSP_K_COUNT] = {};
  int64_t n[TSP_K_COUNT] = {};
  ~ProfState() {  // the thread's timing events, when it ends
    for (hipEvent_t e : pool) (void)hipEventDestroy(e);
    for (const Pending& p : pending) {
      (void)hipEventDestroy(p.a);
      (void)hipEventDestroy(p.b);
    }
  }
};
thread_local ProfState g_prof;

hipError_t prof_event(hipEvent_t* e) {
  if (!g_prof.pool.empty()) {
    *e = g_prof.pool.back();
    g_prof.pool.pop_back();
    return hipSuccess;
  }
  return hipEventCreate(e);
}

// Runs `stmt` (which launches one kernel class on c.s) between two events.
#define TIMED(c, k, stmt)                                              \
  do {                                                                 \
    hipEvent_t ev0_ = nullptr, ev1_ = nullptr;                         \
    if ((c).prof) {                                                    \
      HIP_TRY(prof_event(&ev0_));                                      \
      HIP_TRY(prof_event(&ev1_));                                      \
      HIP_TRY(hipEventRecord(ev0_, (c).s));                            \
    }                                                                  \
    stmt;                                                              \
    if ((c).prof) {                                                    \
      HIP_TRY(hipEventRecord(ev1_, (c).s));                            \
      g_prof.pending.push_back({(k), ev0_, ev1_});                     \
    }                                                                  \
  } while (0)

int begin(Ctx& c, hipStream_t s, hipStream_t cs, uint32_t flags) {
  c.s = s;
  c.prof = (flags & TSP_F_PROFILE) != 0;
  c.side = cs != nullptr && cs != s && !(flags & TSP_F_NO_OVERLAP);
  c.cs = c.side ? cs : s;
  int rc = get_events(&c.ev);
  if (rc) return rc;
  if (c.side) {
    // Copies must not start before earlier work on the compute stream (which
    // produced the inputs or still reads this workspace) is done.
    HIP_TRY(hipEventRecord(c.ev->start, c.s));
    HIP_TRY(hipStreamWaitEvent(c.cs, c.ev->start, 0));
  }
  return TSP_OK;
}

int finish(Ctx& c) {
  if (c.side) {
    HIP_TRY(hipEventRecord(c.ev->join, c.cs));
    HIP_TRY(hipStreamWaitEvent(c.s, c.ev->join, 0));
  }
  return TSP_OK;
}

// Debug modes on the copy stream before a slot is refilled.
int debug_before_fill(Ctx& c, void* slot, size_t bytes) {
  if (c.d->flags & TSP_F_DELAY_COPY) HIP_TRY(launch_spin(20000 /* 200 us */, c.cs));
  if (c.d->flags & TSP_F_POISON_SLOTS)
    HIP_TRY(launch_fill32(slot, c.d->dt == BF16 ? 0x7FC07FC0u : 0x7FC00000u, bytes, c.cs));
  return TSP_OK;
}

// The attention kernels read the other ranks' rows straight from the
// gathered K/V when every zigzag chunk boundary falls on a 64-key tile
// boundary (a tile then comes wholly from the rank's own rows or wholly from
// the others'); otherwise, or when TSP_F_KV_STREAM asks for it, those rows
// are first copied next to the rank's own on the side stream.
bool kv_in_place(const Dims& d) { return d.C % 64 == 0 && !(d.flags & TSP_F_KV_STREAM); }

// Rows of the gathered K/V that rank r needs from the others: its causal
// window is [0, (2D-r)C), minus its own chunks r and 2D-1-r.
// With all_rows, every other rank's rows (positions past the causal window
// as well), so that the slot holds no stale row at all.
int copy_remote_kv(Ctx& c, const char* kv_block, char* slot, bool all_rows = false) {
  const Dims& d = *c.d;
  const size_t es = d.es;
  const int64_t ranges[3][2] = {{0, d.r * d.C},
                                {(d.r + 1) * d.C, (2 * d.D - 1 - d.r) * d.C},
                                {(2 * d.D - d.r) * d.C, all_rows ? d.S : 0}};
  const char* srcK = kv_block;
  const char* srcV = kv_block + kv_v_offset(d) * es;
  char* dstK = slot;
  char* dstV = slot + kv_v_offset(d) * es;
  for (int64_t b = 0; b < d.B; b++)  // sequence b: key rows [b*S, (b+1)*S)
    for (auto& rg : ranges) {
      const int64_t a = b * d.S + rg[0], n = rg[1] - rg[0];
      if (n <= 0) continue;
      const size_t kp = (size_t)d.BS * d.d * es;  // one head's K plane
      HIP_TRY(hipMemcpy2DAsync(dstK + a * d.d * es, kp, srcK + a * d.d * es, kp, n * d.d * es,
                               d.Hkd, hipMemcpyDeviceToDevice, c.cs));
      const size_t vp = (size_t)d.BS * es;  // one V^T row
      HIP_TRY(hipMemcpy2DAsync(dstV + a * es, vp, srcV + a * es, vp, n * es, d.Hkd * d.d,
                               hipMemcpyDeviceToDevice, c.cs));
    }
  return TSP_OK;
}

GemmArgs gemm_base() {
  GemmArgs g;
  memset(&g, 0, sizeof g);
  return g;
}

// QKV projection of this rank's tokens with packed shard w (rows
// [col0, hs + 2ks) of its first block), scattered to Q (if col0 == 0) and to
// K/V at the tokens' global positions, Q and K rotated when rope_theta > 0.
// col0 is 0 or hs.  With np > 1 (col0 == 0), w holds np packed Q|K|V blocks
// back to back; shard u's Q goes to q + u*B*T*hs and its K/V to the kvslot
// block u.
int qkv_gemm(Ctx& c, const void* xn, const char* w, int col0, void* q, char* kvslot, int64_t np = 1) {
  const Dims& d = *c.d;
  GemmArgs g = gemm_base();
  g.A = xn;
  g.lda = d.h;
  g.B = w + (size_t)col0 * d.h * d.es;
  g.ldb = d.h;
  g.M = (int)d.BT;
  g.N = (int)(np * qkv_rows(d) - col0);
  g.K = (int)d.h;
  g.Q = q;
  g.Kd = kvslot;
  g.Vt = kvslot + kv_v_offset(d) * d.es;
  if (np > 1) {
    g.shard_cols = (int)qkv_rows(d);
    g.q_stride = d.BT * d.hs;
    g.kv_stride = (int64_t)kv_block_elems(d);
  }
  g.hs = (int)d.hs;
  g.ks = (int)d.ks;
  g.rope_l2 = d.rope_theta > 0.f ? std::log2((double)d.rope_theta) : 0.0;
  g.hd = (int)d.d;
  g.col0 = col0;
  g.S = d.S;
  g.T = d.T;
  g.batch = (int)d.B;
  g.chunk = d.C;
  g.rank = (int)d.r;
  g.fold = (int)d.D;
  HIP_TRY(launch_gemm(d.dt, EPI_QKV, g, c.s));
  return TSP_OK;
}

// y (+)= a . w^T, or on the last group out = resid + y + a . w^T.
// a [T][ld], w [h][ld]; only the first K columns take part.
int acc_gemm(Ctx& c, const void* a, int64_t lda, int64_t K, int64_t ld, const char* w, float* y, bool first,
             bool last, const void* resid, void* out) {
  const Dims& d = *c.d;
  GemmArgs g = gemm_base();
  g.A = a;
  g.lda = lda;
  g.B = w;
  g.ldb = ld;
  g.M = (int)d.BT;
  g.N = (int)d.h;
  g.K = (int)K;
  g.Y = y;
  g.ldy = d.h;
  g.beta = first ? 0 : 1;
  if (last) {
    g.R = resid;
    g.ldr = d.h;
    g.C = out;
    g.ldc = d.h;
    HIP_TRY(launch_gemm(d.dt, EPI_RESID, g, c.s));
  } else {
    HIP_TRY(launch_gemm(d.dt, EPI_ACC, g, c.s));
  }
  return TSP_OK;
}

// With save_a / save_lse, each head group's attention output goes to
// save_a [B*T][h] (group j at columns j*hs) instead of the workspace, and
// every row's log2 softmax normaliser to save_lse [H][B*T], for the backward.
int attn_body(Ctx& c, const AttnWs& L, const void* x, const void* g1, const void* const* w_attn,
              const void* kv, void* x1, void* save_a = nullptr, float* save_lse = nullptr) {
  const Dims& d = *c.d;
  char* ws = c.ws;
  const size_t es = d.es;
  const size_t qkvbytes = qkv_rows(d) * d.h * es;
  const size_t kvbytes = kv_block_elems(d) * es;
  const int64_t G = acc_group(d), P = launch_shards(d);
  TIMED(c, TSP_K_RMSNORM, HIP_TRY(launch_rmsnorm(d.dt, x, g1, ws + L.xn, d.BT, (int)d.h, d.eps, c.s)));
  // Broadcast iterations j0 .. j0 + np - 1 (shards of ranks j0 ..) per launch.
  for (int64_t j0 = 0, li = 0; j0 < d.D; j0 += P, li++) {
    const int64_t np = std::min<int64_t>(P, d.D - j0);
    const int s = (int)(li & 1);
    const int64_t gi = j0 / G, gp = j0 % G;  // accumulation group, position in it
    const int gb = (int)(gi & 1);
    char* slotw = ws + L.slotw[s];
    char* slotkv = ws + L.slotkv[s];
    char* bo = ws + L.bo[gb];
    // ---- copy stream: receive the shards (Q|K|V into the slot, W_O next to
    // its group's other W_O blocks); the other ranks' K/V rows are read in
    // place from kv, or copied next to the rank's own rows when chunk
    // boundaries do not fall on attention key tiles.  One shard per launch
    // reads the rank's own shard in place.
    if (c.side && li >= 2) HIP_TRY(hipStreamWaitEvent(c.cs, c.ev->freeA[s], 0));
    if (c.side && gp == 0 && gi >= 2) HIP_TRY(hipStreamWaitEvent(c.cs, c.ev->freeO[gb], 0));
    int rc = debug_before_fill(c, slotw, np * qkvbytes);
    if (rc) return rc;
    if (c.d->flags & TSP_F_POISON_SLOTS) {
      const uint32_t nan = d.dt == BF16 ? 0x7FC07FC0u : 0x7FC00000u;
      HIP_TRY(launch_fill32(slotkv, nan, np * kvbytes, c.cs));
      if (gp == 0) HIP_TRY(launch_fill32(bo, nan, (size_t)d.h * G * d.hs * es, c.cs));
    }
    for (int64_t u = 0; u < np; u++) {
      const int64_t j = j0 + u;
      if (np > 1 || j != d.r)
        HIP_TRY(hipMemcpyAsync(slotw + u * qkvbytes, w_attn[j], qkvbytes, hipMemcpyDeviceToDevice, c.cs));
      HIP_TRY(hipMemcpy2DAsync(bo + (gp + u) * d.hs * es, G * d.hs * es, (const char*)w_attn[j] + qkvbytes,
                               d.hs * es, d.hs * es, d.h, hipMemcpyDeviceToDevice, c.cs));
      if (!kv_in_place(d)) {
        rc = copy_remote_kv(c, (const char*)kv + (size_t)j * kvbytes, slotkv + u * kvbytes);
        if (rc) return rc;
      }
    }
    if (c.side) {
      HIP_TRY(hipEventRecord(c.ev->readyA[s], c.cs));
      HIP_TRY(hipStreamWaitEvent(c.s, c.ev->readyA[s], 0));
    }
    // ---- compute stream
    const char* w = np == 1 && j0 == d.r ? (const char*)w_attn[d.r] : slotw;
    TIMED(c, TSP_K_QKV, rc = qkv_gemm(c, ws + L.xn, w, 0, ws + L.q, slotkv, np));
    if (rc) return rc;
    const AttnPlan plan = plan_for(d, np);
    AttnArgs a;
    memset(&a, 0, sizeof a);
    a.Q = ws + L.q;
    a.K = slotkv;
    a.Vt = slotkv + kv_v_offset(d) * es;
    if (kv_in_place(d)) {
      const char* kvj = (const char*)kv + (size_t)j0 * kvbytes;
      a.Kg = kvj;
      a.Vtg = kvj + kv_v_offset(d) * es;
    }
    if (np > 1) {
      a.kvh_per_shard = (int)d.Hkd;
      a.shard_stride = (int64_t)kv_block_elems(d);
    }
    // these shards' columns of the group's [B*T][G*hs], or of save_a
    char* const obase = save_a ? (char*)save_a + gi * G * d.hs * es : ws + L.o;
    const int64_t ldA = save_a ? d.h : G * d.hs;
    a.O = obase + gp * d.hs * es;
    if (save_lse) a.LSE = save_lse + j0 * d.Hd * d.BT;
    a.Op = (float*)(ws + L.op);
    a.ML = (float*)(ws + L.ml);
    a.T = d.T;
    a.S = d.S;
    a.batch = (int)d.B;
    a.chunk = d.C;
    a.ldo = (int)ldA;
    a.rank = (int)d.r;
    a.fold = (int)d.D;
    a.Hd = (int)(np * d.Hd);
    a.grp = (int)(d.H / d.Hkv);
    a.bq = plan.bq;
    a.nqt = plan.nqt;
    a.lseg = plan.lseg;
    a.maxseg = plan.maxseg;
    a.nitems = plan.nitems;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d.d));
    // Largest block sum of exponentials before the softmax reference is
    // raised: 2^64 keeps every term far from fp32/bf16 overflow.
    a.sum_cap = (d.flags & TSP_F_RESCALE_TEST) ? 2.0f : 18446744073709551616.0f;
    TIMED(c, TSP_K_ATTN, HIP_TRY(launch_attention(d.dt, (int)d.d, a, plan, 0, c.s)));
    if (plan.split) TIMED(c, TSP_K_MERGE, HIP_TRY(launch_attention(d.dt, (int)d.d, a, plan, 1, c.s)));
    if (gp + np == G || j0 + np == d.D) {  // group complete: one O projection over its shards
      TIMED(c, TSP_K_OPROJ,
            rc = acc_gemm(c, obase, ldA, (gp + np) * d.hs, G * d.hs, bo, (float*)(ws + L.y), gi == 0,
                          j0 + np == d.D, x, x1));
      if (rc) return rc;
      if (c.side) HIP_TRY(hipEventRecord(c.ev->freeO[gb], c.s));
    }
    if (c.side) HIP_TRY(hipEventRecord(c.ev->freeA[s], c.s));
  }
  return TSP_OK;
}

int mlp_body(Ctx& c, const MlpWs& L, const void* x1, const void* g2, const void* const* w_mlp,
             void* out) {
  const Dims& d = *c.d;
  char* ws = c.ws;
  const size_t es = d.es;
  const size_t wbytes = (size_t)d.Fs * d.h * es;  // one shard's W1 (or W3) block
  const int64_t G = acc_group(d), P = launch_shards(d);
  TIMED(c, TSP_K_RMSNORM, HIP_TRY(launch_rmsnorm(d.dt, x1, g2, ws + L.xn, d.BT, (int)d.h, d.eps, c.s)));
  // Two consecutive launch groups of one accumulation group share one W1/W3
  // launch (their slots as the two weight blocks of the SwiGLU GEMM): the
  // second group's shards are in by then at the measured shapes, and one
  // launch over both fills the CUs' last round of tiles once, not twice.
  struct Pending {
    const char* b;
    int64_t n, gp;
    int s;
  } pend = {nullptr, 0, 0, -1};
  // Ring steps t0 .. t0 + np - 1 (shards (r + t) mod D) per launch.
  for (int64_t t0 = 0, li = 0; t0 < d.D; t0 += P, li++) {
    const int64_t np = std::min<int64_t>(P, d.D - t0);
    const int s = (int)(li & 1);
    const int64_t gi = t0 / G, gp = t0 % G;
    const int gb = (int)(gi & 1);
    char* bw = ws + L.bw[gb];
    const char* w = (const char*)w_mlp[d.r];
    // ---- copy stream: W1|W3 of the launch's shards into the slot (the own
    // shard is read in place when it runs alone); every shard's W2 block
    // next to its group's others.  With one shard per launch, ring step 0
    // uses no slot, so slot 0 is first refilled at step 2 and slot 1 at 3.
    const bool slot_reused = np == 1 && P == 1 ? t0 >= 3 : li >= 2;
    if (c.side && slot_reused) HIP_TRY(hipStreamWaitEvent(c.cs, c.ev->freeM[s], 0));
    if (c.side && gp == 0 && gi >= 2) HIP_TRY(hipStreamWaitEvent(c.cs, c.ev->freeW[gb], 0));
    if (P > 1 || t0 > 0) {
      char* slotw = ws + L.slotw[s];
      int rc = debug_before_fill(c, slotw, 2 * np * wbytes);
      if (rc) return rc;
      for (int64_t u = 0; u < np; u++) {
        const char* src = (const char*)w_mlp[(d.r + t0 + u) % d.D];
        HIP_TRY(hipMemcpyAsync(slotw + u * wbytes, src, wbytes, hipMemcpyDeviceToDevice, c.cs));
        HIP_TRY(hipMemcpyAsync(slotw + (np + u) * wbytes, src + wbytes, wbytes, hipMemcpyDeviceToDevice, c.cs));
      }
      w = slotw;
    }
    if ((c.d->flags & TSP_F_POISON_SLOTS) && gp == 0)
      HIP_TRY(launch_fill32(bw, d.dt == BF16 ? 0x7FC07FC0u : 0x7FC00000u,
                            (size_t)d.h * G * d.Fs * es, c.cs));
    for (int64_t u = 0; u < np; u++) {
      const char* src = (const char*)w_mlp[(d.r + t0 + u) % d.D];
      HIP_TRY(hipMemcpy2DAsync(bw + (gp + u) * d.Fs * es, G * d.Fs * es, src + 2 * wbytes, d.Fs * es,
                               d.Fs * es, d.h, hipMemcpyDeviceToDevice, c.cs));
    }
    if (c.side) {
      HIP_TRY(hipEventRecord(c.ev->readyM[s], c.cs));
      HIP_TRY(hipStreamWaitEvent(c.s, c.ev->readyM[s], 0));
    }
    // ---- compute stream
    if (TSP_W13_PAIR && P > 1 && pend.s < 0 && gp + np < G && t0 + np < d.D) {
      pend = {w, np, gp, s};  // W1/W3 runs with the next launch group's
      continue;
    }
    GemmArgs g = gemm_base();
    g.A = ws + L.xn;
    g.lda = d.h;
    g.B = w;
    g.B3 = w + np * wbytes;
    g.ldb = d.h;
    g.M = (int)d.BT;
    g.N = (int)(np * d.Fs);
    g.K = (int)d.h;
    g.C = ws + L.gg + gp * d.Fs * es;  // these shards' columns of the group's [T][G*Fs]
    g.ldc = G * d.Fs;
    if (pend.s >= 0) {  // the previous launch group's shards first (columns just before these)
      g.B_2 = g.B;
      g.B3_2 = g.B3;
      g.B = pend.b;
      g.B3 = pend.b + pend.n * wbytes;
      g.n_split = (int)(pend.n * d.Fs);
      g.N += g.n_split;
      g.C = ws + L.gg + pend.gp * d.Fs * es;
    }
    TIMED(c, TSP_K_W13, HIP_TRY(launch_gemm(d.dt, EPI_SWIGLU, g, c.s)));
    int rc = 0;
    if (gp + np == G || t0 + np == d.D) {  // group complete: one W2 projection over its shards
      TIMED(c, TSP_K_W2,
            rc = acc_gemm(c, ws + L.gg, G * d.Fs, (gp + np) * d.Fs, G * d.Fs, bw, (float*)(ws + L.y), gi == 0,
                          t0 + np == d.D, x1, out));
      if (rc) return rc;
      if (c.side) HIP_TRY(hipEventRecord(c.ev->freeW[gb], c.s));
    }
    if (c.side) {
      HIP_TRY(hipEventRecord(c.ev->freeM[s], c.s));
      if (pend.s >= 0) HIP_TRY(hipEventRecord(c.ev->freeM[pend.s], c.s));
    }
    pend.s = -1;
  }
  return TSP_OK;
}

int check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps) {
    if (!p) return fail(TSP_E_INVAL, "a required pointer is NULL");
    if (!aligned(p)) return fail(TSP_E_ALIGN, "pointer %p is not 16-byte aligned", p);
  }
  return TSP_OK;
}

int check_shards(const void* const* w, int64_t D, const char* what) {
  if (!w) return fail(TSP_E_INVAL, "%s pointer array is NULL", what);
  for (int64_t j = 0; j < D; j++) {
    if (!w[j]) return fail(TSP_E_INVAL, "%s[%lld] is NULL", what, (long long)j);
    if (!aligned(w[j])) return fail(TSP_E_ALIGN, "%s[%lld] is not 16-byte aligned", what, (long long)j);
  }
  return TSP_OK;
}

// ---- backward of the MLP half -------------------------------------------
// Workspace: the recomputed n2 and its transpose, dout transposed, the fp32
// products [a | b] = n2 [W1 | W3] (one GEMM over the shard's contiguous W1|W3
// block) and dg = dout W2 of one shard, [da | db]
// and g = silu(a) b with their transposes, the shard's W2 and W1|W3 blocks
// transposed, the fp32 gradient of n2 and the per-row rstd.
struct MlpBwdWs {
  size_t n2, n2t, dot, ab, dg, dab, dabt, gm, gmt, w2t, w13t, dn, rs, end;
};

// Attention-core backward: the recomputed forward output of the group, the
// per-row log-sum-exp and rowsum(dO * O), and the forward's split partials.
// Transposed copies for the backward kernels: Q and dO [d][Hd][B][Tp], K
// [d][Hkd][B][Sp] (each sequence padded with zeros to a multiple of 64
// rows), V by rows [B*S][Hkd * d].
int64_t pad64(int64_t n) { return (n + 63) / 64 * 64; }
struct AttnBwdWs {
  size_t o, lse, dl, qt, dot, kt, vr, dqp, op, ml, end;
  int dq_seg, dq_items;  // the dQ kernel's key segments (attn_bwd_dq_plan)
};
AttnBwdWs attn_bwd_ws(const Dims& d, size_t base = 0) {
  AttnBwdWs w;
  size_t o = base;
  w.o = o; o += al((size_t)d.BT * d.hs * d.es);
  w.lse = o; o += al((size_t)d.Hd * d.BT * 4);
  w.dl = o; o += al((size_t)d.Hd * d.BT * 4);
  w.qt = o; o += al((size_t)d.d * d.Hd * d.B * pad64(d.T) * d.es);
  w.dot = o; o += al((size_t)d.d * d.Hd * d.B * pad64(d.T) * d.es);
  w.kt = o; o += al((size_t)d.d * d.Hkd * d.B * pad64(d.S) * d.es);
  w.vr = o; o += al((size_t)d.d * d.Hkd * d.BS * d.es);
  attn_bwd_dq_plan(d.T, d.C, (int)d.r, (int)d.D, d.Hd * d.B, &w.dq_seg, &w.dq_items);
  w.dqp = o; o += al((size_t)d.Hd * d.B * w.dq_items * 128 * d.d * 4);  // 128-row query blocks
  const AttnPlan p = plan_of(d);
  const size_t nslot = p.split ? (size_t)d.Hd * d.B * p.nqt * p.maxseg * p.bq : 0;
  w.op = o; o += al(nslot * d.d * 4);
  w.ml = o; o += al(nslot * 2 * 4);
  w.end = o;
  return w;
}

MlpBwdWs mlp_bwd_ws(const Dims& d, size_t base = 0) {
  MlpBwdWs w;
  size_t o = base;
  const size_t T = d.BT, h = d.h, F = d.Fs, es = d.es;
  w.n2 = o; o += al(T * h * es);
  w.n2t = o; o += al(T * h * es);
  w.dot = o; o += al(T * h * es);
  w.ab = o; o += al(T * 2 * F * 4);
  w.dg = o; o += al(T * F * 4);
  w.dab = o; o += al(T * 2 * F * es);
  w.dabt = o; o += al(T * 2 * F * es);
  w.gm = o; o += al(T * F * es);
  w.gmt = o; o += al(T * F * es);
  w.w2t = o; o += al(F * h * es);
  w.w13t = o; o += al(2 * F * h * es);
  w.dn = o; o += al(T * h * 4);
  w.rs = o; o += al(T * 4);
  w.end = o;
  return w;
}

// y = a . b^T in fp32 (a [M][K] pitch lda, b [N][K] pitch ldb), or y += when accumulate.
int plain_gemm(Ctx& c, const void* a, int64_t lda, const void* b, int64_t ldb, int64_t M, int64_t N,
               int64_t K, float* y, int64_t ldy, bool accumulate) {
  GemmArgs g = gemm_base();
  g.A = a;
  g.lda = lda;
  g.B = b;
  g.ldb = ldb;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.Y = y;
  g.ldy = ldy;
  g.beta = accumulate ? 1 : 0;
  HIP_TRY(launch_gemm(c.d->dt, EPI_ACC, g, c.s));
  return TSP_OK;
}

int mlp_bwd_body(Ctx& c, const MlpBwdWs& L, const void* x1, const void* g2, const void* const* w_mlp,
                 const void* dout, void* dx1, float* dg2, float* const* dw_mlp) {
  const Dims& d = *c.d;
  char* ws = c.ws;
  const int64_t T = d.BT, h = d.h, F = d.Fs;
  const size_t es = d.es;
  float* fab = (float*)(ws + L.ab);
  float* fdg = (float*)(ws + L.dg);
  float* dn = (float*)(ws + L.dn);
  HIP_TRY(launch_rmsnorm(d.dt, x1, g2, ws + L.n2, T, (int)h, d.eps, c.s));
  HIP_TRY(launch_transpose(d.dt, ws + L.n2, ws + L.n2t, T, h, h, T, c.s));
  HIP_TRY(launch_transpose(d.dt, dout, ws + L.dot, T, h, h, T, c.s));
  HIP_TRY(launch_fill32(dg2, 0u, (size_t)h * 4, c.s));
  int rc = 0;
  for (int64_t t = 0; t < d.D; t++) {  // the ring order of the forward: own shard first
    const int64_t j = (d.r + t) % d.D;
    const char* w1 = (const char*)w_mlp[j];
    const char* w2 = w1 + 2 * (size_t)F * h * es;  // [h][F]
    if ((rc = plain_gemm(c, ws + L.n2, h, w1, h, T, 2 * F, h, fab, 2 * F, false))) return rc;
    HIP_TRY(launch_transpose(d.dt, w2, ws + L.w2t, h, F, F, h, c.s));
    if ((rc = plain_gemm(c, dout, h, ws + L.w2t, h, T, F, h, fdg, F, false))) return rc;
    HIP_TRY(launch_swiglu_bwd(d.dt, fab, fdg, ws + L.dab, ws + L.gm, T, F, c.s));
    // dn2 (+)= [da | db] . [W1; W3]  (B operand: the W1|W3 block transposed)
    HIP_TRY(launch_transpose(d.dt, w1, ws + L.w13t, 2 * F, h, h, 2 * F, c.s));
    if ((rc = plain_gemm(c, ws + L.dab, 2 * F, ws + L.w13t, 2 * F, T, h, 2 * F, dn, h, t > 0))) return rc;
    // this rank's partial weight gradients of shard j, in the shard's layout
    HIP_TRY(launch_transpose(d.dt, ws + L.dab, ws + L.dabt, T, 2 * F, 2 * F, T, c.s));
    HIP_TRY(launch_transpose(d.dt, ws + L.gm, ws + L.gmt, T, F, F, T, c.s));
    if ((rc = plain_gemm(c, ws + L.dabt, T, ws + L.n2t, T, 2 * F, h, T, dw_mlp[j], h, false))) return rc;
    if ((rc = plain_gemm(c, ws + L.dot, T, ws + L.gmt, T, h, F, T, dw_mlp[j] + 2 * F * h, F, false)))
      return rc;
  }
  // the gain's partial sums go to n2t, free once the last shard's GEMMs have read it
  // (T h es bytes hold ceil(T / 64) h floats for every T >= 2)
  HIP_TRY(launch_rmsnorm_bwd(d.dt, x1, g2, dn, dout, dx1, (float*)(ws + L.rs), dg2, (float*)(ws + L.n2t), T,
                             (int)h, d.eps, c.s));
  return TSP_OK;
}

// ---- whole-layer backward workspaces ---------------------------------------
// Part 1 (MLP half, then per head group the attention core and W_O): n1, dx1
// transposed, the group's rotated Q and complete K/V slot, its output O
// transposed, W_O's block transposed and dA; then the MLP backward's and the
// attention-core backward's regions, which are used one after the other and
// share their space.
struct LayerBwdWs {
  size_t n1, dx1t, q, slotkv, ot, wot, da, shared, end;
  MlpBwdWs mlp;
  AttnBwdWs attn;
};
LayerBwdWs layer_bwd_ws(const Dims& d) {
  LayerBwdWs w;
  size_t o = 0;
  const size_t es = d.es;
  w.n1 = o; o += al((size_t)d.BT * d.h * es);
  w.dx1t = o; o += al((size_t)d.h * d.BT * es);
  w.q = o; o += al((size_t)d.Hd * d.BT * d.d * es);
  w.slotkv = o; o += al(kv_block_elems(d) * es);
  w.ot = o; o += al((size_t)d.hs * d.BT * es);
  w.wot = o; o += al((size_t)d.hs * d.h * es);
  w.da = o; o += al((size_t)d.BT * d.hs * es);
  w.shared = o;
  w.mlp = mlp_bwd_ws(d, o);
  w.attn = attn_bwd_ws(d, o);
  w.end = std::max(w.mlp.end, w.attn.end);
  return w;
}
// Part 2 (after the reduce-scatter of dK/dV): n1 and its transpose, one
// shard's [dQ | dK | dV] and its transpose, the shard's Q|K|V block
// transposed, dn1 (fp32) and the per-row rstd.
struct LayerBwd2Ws {
  size_t n1, n1t, g, gt, wt, dn, rs, end;
};
LayerBwd2Ws layer_bwd2_ws(const Dims& d) {
  LayerBwd2Ws w;
  size_t o = 0;
  const size_t es = d.es, N = qkv_rows(d);
  w.n1 = o; o += al((size_t)d.BT * d.h * es);
  w.n1t = o; o += al((size_t)d.h * d.BT * es);
  w.g = o; o += al((size_t)d.BT * N * es);
  w.gt = o; o += al(N * d.BT * es);
  w.wt = o; o += al((size_t)d.h * N * es);
  w.dn = o; o += al((size_t)d.BT * d.h * 4);
  w.rs = o; o += al((size_t)d.BT * 4);
  w.end = o;
  return w;
}

// ---- attention-core backward pieces ----------------------------------------
int check_attn_bwd_dims(const Dims& d) {
  if (d.dt != BF16) return fail(TSP_E_DTYPE, "the attention backward runs in bf16 only");
  if (d.d != 64 && d.d != 128) return fail(TSP_E_SHAPE, "the attention backward needs head_dim 64 or 128");
  return TSP_OK;
}

AttnArgs attn_args(const Dims& d, const AttnPlan& plan) {
  AttnArgs a;
  memset(&a, 0, sizeof a);
  a.T = d.T;
  a.S = d.S;
  a.batch = (int)d.B;
  a.chunk = d.C;
  a.rank = (int)d.r;
  a.fold = (int)d.D;
  a.Hd = (int)d.Hd;
  a.grp = (int)(d.H / d.Hkv);
  a.bq = plan.bq;
  a.nqt = plan.nqt;
  a.lseg = plan.lseg;
  a.maxseg = plan.maxseg;
  a.nitems = plan.nitems;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d.d));
  a.sum_cap = 18446744073709551616.0f;
  return a;
}

// The group's attention output O [B*T][hs] and per-row log-sum-exp, from its
// rotated queries q and every position's K / V^T in kv.
int attn_recompute(Ctx& c, const AttnBwdWs& L, const void* q, const void* kv) {
  const Dims& d = *c.d;
  const AttnPlan plan = plan_of(d);
  AttnArgs a = attn_args(d, plan);
  a.Q = q;
  a.K = kv;
  a.Vt = (const char*)kv + kv_v_offset(d) * d.es;
  a.O = c.ws + L.o;
  a.Op = (float*)(c.ws + L.op);
  a.ML = (float*)(c.ws + L.ml);
  a.LSE = (float*)(c.ws + L.lse);
  a.ldo = (int)d.hs;
  HIP_TRY(launch_attention(d.dt, (int)d.d, a, plan, 0, c.s));
  if (plan.split) HIP_TRY(launch_attention(d.dt, (int)d.d, a, plan, 1, c.s));
  return TSP_OK;
}

// dq [Hd][B*T][d] and this rank's partial dk, dv [Hkd][B*S][d] (fp32) of the
// group, given its forward output o [B*T][ldo_fwd], the rows' log2 softmax
// normalisers lse [Hd][B*T] and dout [B*T][ldo].
int attn_core_grads(Ctx& c, const AttnBwdWs& L, const void* q, const void* kv, const void* o, int ldo_fwd,
                    const float* lse, const void* dout, int ldo, float* dq, float* dk, float* dv) {
  const Dims& d = *c.d;
  const hipStream_t s = c.s;
  char* w = c.ws;
  const void* vt = (const char*)kv + kv_v_offset(d) * d.es;
  AttnBwdArgs b;
  memset(&b, 0, sizeof b);
  b.Q = q;
  b.K = kv;
  b.Vt = vt;
  b.O = o;
  b.dO = dout;
  b.LSE = lse;
  b.Dl = (float*)(w + L.dl);
  b.dQ = dq;
  b.dK = dk;
  b.dV = dv;
  b.T = d.T;
  b.S = d.S;
  b.chunk = d.C;
  b.ldo = ldo;
  b.ldo_fwd = ldo_fwd;
  b.rank = (int)d.r;
  b.fold = (int)d.D;
  b.batch = (int)d.B;
  b.grp = (int)(d.H / d.Hkv);
  b.Hd = (int)d.Hd;
  b.Hkd = (int)d.Hkd;
  b.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d.d));
  b.scale = (float)(1.0 / std::sqrt((double)d.d));
  b.dQp = (float*)(w + L.dqp);
  b.dq_seg = L.dq_seg;
  b.dq_items = L.dq_items;
  b.Tp = pad64(d.T);
  b.Sp = pad64(d.S);
  b.Qt = w + L.qt;
  b.dOt = w + L.dot;
  b.Kt = w + L.kt;
  b.Vr = w + L.vr;
  // matrix z = t * B + b of each transposed copy is head (or K/V head) t, sequence b
  HIP_TRY(launch_transpose_pad(d.dt, q, w + L.qt, d.T, b.Tp, d.d, d.d, d.Hd * d.B * b.Tp, d.Hd * d.B, d.B,
                               d.BT * d.d, d.T * d.d, s));
  HIP_TRY(launch_transpose_pad(d.dt, dout, w + L.dot, d.T, b.Tp, d.d, ldo, d.Hd * d.B * b.Tp, d.Hd * d.B, d.B,
                               d.d, d.T * ldo, s));
  HIP_TRY(launch_transpose_pad(d.dt, kv, w + L.kt, d.S, b.Sp, d.d, d.d, d.Hkd * d.B * b.Sp, d.Hkd * d.B, d.B,
                               d.BS * d.d, d.S * d.d, s));
  HIP_TRY(launch_transpose(d.dt, vt, w + L.vr, d.Hkd * d.d, d.BS, d.BS, d.Hkd * d.d, s));
  for (int part = 0; part < 3; part++) HIP_TRY(launch_attn_bwd((int)d.d, b, part, s));
  return TSP_OK;
}

// ---- the allocation-free layer entry point --------------------------------
// Its workspace is this file-scope device array, one copy per GPU, held from
// module load until the process ends.  Host code never names it directly
// (the name is a host-side stand-in, not a device address): the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current, and is kept per device.
static __device__ __attribute__((aligned(256))) char scratch[TSP_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDev] = {};

int scratch_ptr(void** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDev) return fail(TSP_E_HIP, "device index %d unsupported", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(TSP_E_HIP, "hipGetSymbolAddress returned a null scratch address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TSP_OK;
}

}  // namespace

extern "C" {

size_t tsp_workspace_bytes(const tsp_dims* dims, int which) {
  Dims d;
  if (check_dims(dims, &d)) return 0;
  switch (which) {
    case TSP_WS_ATTN: return attn_ws(d, 0).end;
    case TSP_WS_MLP: return mlp_ws(d, 0).end;
    case TSP_WS_LAYER: {
      const size_t x1 = al((size_t)d.BT * d.h * d.es);
      const AttnWs a = attn_ws(d, x1);
      return mlp_ws(d, a.end).end;
    }
    case TSP_WS_KV: return kv_ws_bytes(d);
    case TSP_WS_MLP_BWD: return mlp_bwd_ws(d).end;
    case TSP_WS_ATTN_BWD: return attn_bwd_ws(d).end;
    case TSP_WS_LAYER_BWD: return layer_bwd_ws(d).end;
    case TSP_WS_LAYER_BWD_FINISH: return layer_bwd2_ws(d).end;
    default: return 0;
  }
}

const char* tsp_strerror(int status) {
  switch (status) {
    case TSP_OK: return "success";
    case TSP_E_INVAL: return "invalid argument";
    case TSP_E_SHAPE: return "unsupported shape";
    case TSP_E_ALIGN: return "pointer not 16-byte aligned";
    case TSP_E_WORKSPACE: return "workspace too small";
    case TSP_E_DTYPE: return "unsupported dtype";
    case TSP_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* tsp_last_error(void) { return g_err.c_str(); }

int tsp_zigzag_positions(int64_t seq, int32_t fold, int32_t rank, int64_t* out) {
  if (fold <= 0 || rank < 0 || rank >= fold || seq < 0 || (!out && seq > 0))
    return fail(TSP_E_INVAL, "bad zigzag arguments");
  if (seq % (2 * (int64_t)fold)) return fail(TSP_E_SHAPE, "seq is not a multiple of 2*fold");
  const int64_t C = seq / (2 * fold);
  for (int64_t i = 0; i < C; i++) {
    out[i] = rank * C + i;
    out[C + i] = (int64_t)(2 * fold - 1 - rank) * C + i;
  }
  return TSP_OK;
}

int tsp_attn_shard(const tsp_dims* dims, const void* x, const void* g1, const void* const* w_attn,
                   const void* kv, void* x1, void* ws, size_t ws_bytes, void* stream,
                   void* copy_stream) {
  g_err.clear();
  Dims d;
  int rc = check_dims(dims, &d);
  if (rc) return rc;
  if (d.S == 0) return TSP_OK;
  if ((rc = check_ptrs({x, g1, kv, x1, ws})) || (rc = check_shards(w_attn, d.D, "w_attn"))) return rc;
  const AttnWs L = attn_ws(d, 0);
  if (ws_bytes < L.end)
    return fail(TSP_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.end);
  Ctx c{&d, (char*)ws};
  if ((rc = begin(c, (hipStream_t)stream, (hipStream_t)copy_stream, d.flags))) return rc;
  if ((rc = attn_body(c, L, x, g1, w_attn, kv, x1))) return rc;
  return finish(c);
}

int tsp_attn_shard_save(const tsp_dims* dims, const void* x, const void* g1, const void* const* w_attn,
                        const void* kv, void* x1, void* attn_out, float* lse, void* ws, size_t ws_bytes,
                        void* stream, void* copy_stream) {
  g_err.clear();
  Dims d;
  int rc = check_dims(dims, &d);
  if (rc) return rc;
  if (d.S == 0) return TSP_OK;
  if ((rc = check_ptrs({x, g1, kv, x1, attn_out, lse, ws})) || (rc = check_shards(w_attn, d.D, "w_attn")))
    return rc;
  const AttnWs L = attn_ws(d, 0);
  if (ws_bytes < L.end)
    return fail(TSP_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.end);
  Ctx c{&d, (char*)ws};
  if ((rc = begin(c, (hipStream_t)stream, (hipStream_t)copy_stream, d.flags))) return rc;
  if ((rc = attn_body(c, L, x, g1, w_attn, kv, x1, attn_out, lse))) return rc;
  return finish(c);
}

int tsp_mlp_shard(const tsp_dims* dims, const void* x1, const void* g2, const void* const* w_mlp,
                  void* out, void* ws, size_t ws_bytes, void* stream, void* copy_stream) {
  g_err.clear();
  Dims d;
  int rc = check_dims(dims, &d);
  if (rc) return rc;
  if (d.S == 0) return TSP_OK;
  if ((rc = check_ptrs({x1, g2, out, ws})) || (rc = check_shards(w_mlp, d.D, "w_mlp"))) return rc;
  const MlpWs L = mlp_ws(d, 0);
  if (ws_bytes < L.end)
    return fail(TSP_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.end);
  Ctx c{&d, (char*)ws};
  if ((rc = begin(c, (hipStream_t)stream, (hipStream_t)copy_stream, d.flags))) return rc;
  if ((rc = mlp_body(c, L, x1, g2, w_mlp, out))) return rc;
  return finish(c);
}

int tsp_mlp_shard_backward(const tsp_dims* dims, const void* x1, const void* g2,
                           const void* const* w_mlp, const void* dout, void* dx1, float* dg2,
                           float* const* dw_mlp, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  Dims d;
  int rc = check_dims(dims, &d);
  if (rc) return rc;
  if (d.S == 0) return TSP_OK;
  if ((rc = check_ptrs({x1, g2, dout, dx1, dg2, ws})) || (rc = check_shards(w_mlp, d.D, "w_mlp")) ||
      (rc = check_shards((const void* const*)dw_mlp, d.D, "dw_mlp")))
    return rc;
  const MlpBwdWs L = mlp_bwd_ws(d);
  if (ws_bytes < L.end)
    return fail(TSP_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.end);
  Ctx c{&d, (char*)ws, (hipStream_t)stream, (hipStream_t)stream, false, nullptr, false};
  return mlp_bwd_body(c, L, x1, g2, w_mlp, dout, dx1, dg2, dw_mlp);
}

int tsp_layer_shard(const tsp_dims* dims, const void* x, const void* g1, const void* const* w_attn,
                    const void* kv, const void* g2, const void* const* w_mlp, void* out, void* ws,
                    size_t ws_bytes, void* stream, void* copy_stream) {
  g_err.clear();
  Dims d;
  int rc = check_dims(dims, &d);
  if (rc) return rc;
  if (d.S == 0) return TSP_OK;
  if ((rc = check_ptrs({x, g1, kv, g2, out, ws})) || (rc = check_shards(w_attn, d.D, "w_attn")) ||
      (rc = check_shards(w_mlp, d.D, "w_mlp")))
    return rc;
  const size_t x1off = 0;
  const AttnWs A = attn_ws(d, al((size_t)d.BT * d.h * d.es));
  const MlpWs M = mlp_ws(d, A.end);
  if (ws_bytes < M.end) return fail(TSP_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, M.end);
  Ctx c{&d, (char*)ws};
  if ((rc = begin(c, (hipStream_t)stream, (hipStream_t)copy_stream, d.flags))) return rc;
  void* x1 = (char*)ws + x1off;
  if ((rc = attn_body(c, A, x, g1, w_attn, kv, x1))) return rc;
  if ((rc = mlp_body(c, M, x1, g2, w_mlp, out))) return rc;
  return finish(c);
}

int tsp_layer_shard_noalloc(const tsp_dims* dims, const void* x, const void* g1, const void* const* w_attn,
                            const void* kv, const void* g2, const void* const* w_mlp, void* out, void* stream,
                            void* copy_stream) {
  g_err.clear();
  Dims d;
  int rc = check_dims(dims, &d);
  if (rc) return rc;
  if (d.S == 0) return TSP_OK;
  if (d.flags & TSP_F_PROFILE)
    return fail(TSP_E_INVAL, "TSP_F_PROFILE creates timing events per launch; use tsp_layer_shard to profile");
  if ((rc = check_ptrs({x, g1, kv, g2, out})) || (rc = check_shards(w_attn, d.D, "w_attn")) ||
      (rc = check_shards(w_mlp, d.D, "w_mlp")))
    return rc;
  const AttnWs A = attn_ws(d, al((size_t)d.BT * d.h * d.es));
  const MlpWs M = mlp_ws(d, A.end);
  if (M.end > (size_t)TSP_NOALLOC_SCRATCH_BYTES)
    return fail(TSP_E_WORKSPACE, "this layer needs %zu bytes of scratch; the static scratch holds %llu",
                M.end, (unsigned long long)TSP_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((rc = scratch_ptr(&ws))) return rc;
  Ctx c{&d, (char*)ws};
  if ((rc = begin(c, (hipStream_t)stream, (hipStream_t)copy_stream, d.flags))) return rc;
  void* x1 = ws;  // x1 first, as in tsp_layer_shard's workspace
  if ((rc = attn_body(c, A, x, g1, w_attn, kv, x1))) return rc;
  if ((rc = mlp_body(c, M, x1, g2, w_mlp, out))) return rc;
  return finish(c);
}

int tsp_layer_shard_backward(const tsp_dims* dims, const void* x, const void* x1, const void* g1,
                             const void* const* w_attn, const void* kv, const void* g2, const void* const* w_mlp,
                             const void* dout, const void* attn_saved, const float* lse_saved, void* dx1,
                             float* dg2, float* const* dw_mlp, float* const* dw_o, float* dq, float* dkv, void* ws,
                             size_t ws_bytes, void* stream) {
  g_err.clear();
  Dims d;
  int rc = check_dims(dims, &d);
  if (rc) return rc;
  if (d.S == 0) return TSP_OK;
  if ((rc = check_attn_bwd_dims(d))) return rc;
  if (!attn_saved != !lse_saved)
    return fail(TSP_E_INVAL, "attn_saved and lse_saved are given together or not at all");
  if ((rc = check_ptrs({x, x1, g1, kv, g2, dout, dx1, dg2, dq, dkv, ws})) ||
      (rc = check_shards(w_attn, d.D, "w_attn")) || (rc = check_shards(w_mlp, d.D, "w_mlp")) ||
      (rc = check_shards((const void* const*)dw_mlp, d.D, "dw_mlp")) ||
      (rc = check_shards((const void* const*)dw_o, d.D, "dw_o")))
    return rc;
  const LayerBwdWs L = layer_bwd_ws(d);
  if (ws_bytes < L.end) return fail(TSP_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.end);
  Ctx c{&d, (char*)ws, (hipStream_t)stream, (hipStream_t)stream, false, nullptr, false};
  char* w = c.ws;
  const size_t es = d.es;
  // MLP half: dx1, the gain's and every MLP shard's partial gradient
  if ((rc = mlp_bwd_body(c, L.mlp, x1, g2, w_mlp, dout, dx1, dg2, dw_mlp))) return rc;
  HIP_TRY(launch_rmsnorm(d.dt, x, g1, w + L.n1, d.BT, (int)d.h, d.eps, c.s));
  HIP_TRY(launch_transpose(d.dt, dx1, w + L.dx1t, d.BT, d.h, d.h, d.BT, c.s));
  const size_t qkvbytes = qkv_rows(d) * d.h * es;
  const size_t kvbytes = kv_block_elems(d) * es;
  const double l2c = d.rope_theta > 0.f ? std::log2((double)d.rope_theta) / (double)d.d : 0.0;
  for (int64_t j = 0; j < d.D; j++) {  // head group j, in broadcast order
    const char* wj = (const char*)w_attn[j];
    float* dqj = dq + (size_t)j * d.Hd * d.BT * d.d;
    float* dkj = dkv + (size_t)j * kv_block_elems(d);
    float* dvj = dkj + kv_v_offset(d);
    // the group's rotated Q, and its K/V complete: own rows projected here,
    // every other rank's rows copied from the gathered buffer
    if ((rc = copy_remote_kv(c, (const char*)kv + (size_t)j * kvbytes, w + L.slotkv, true))) return rc;
    if ((rc = qkv_gemm(c, w + L.n1, wj, 0, w + L.q, w + L.slotkv))) return rc;
    // the group's attention output and normalisers: the forward's, or recomputed
    const void* oj = w + L.attn.o;
    const float* lj = (const float*)(w + L.attn.lse);
    int64_t ldoj = d.hs;
    if (attn_saved) {
      oj = (const char*)attn_saved + (size_t)j * d.hs * es;
      lj = lse_saved + (size_t)j * d.Hd * d.BT;
      ldoj = d.h;
    } else if ((rc = attn_recompute(c, L.attn, w + L.q, w + L.slotkv))) {
      return rc;
    }
    // dA = dx1 W_O^T, and this rank's partial dW_O = dx1^T A (packed layout)
    HIP_TRY(launch_transpose(d.dt, wj + qkvbytes, w + L.wot, d.h, d.hs, d.hs, d.h, c.s));
    GemmArgs g = gemm_base();
    g.A = dx1;
    g.lda = d.h;
    g.B = w + L.wot;
    g.ldb = d.h;
    g.M = (int)d.BT;
    g.N = (int)d.hs;
    g.K = (int)d.h;
    g.C = w + L.da;
    g.ldc = d.hs;
    HIP_TRY(launch_gemm(d.dt, EPI_STORE, g, c.s));
    HIP_TRY(launch_transpose(d.dt, oj, w + L.ot, d.BT, d.hs, ldoj, d.BT, c.s));
    if ((rc = plain_gemm(c, w + L.dx1t, d.BT, w + L.ot, d.BT, d.h, d.hs, d.BT, dw_o[j], d.hs, false))) return rc;
    // the attention core: dQ of the rank's rows, partial dK / dV of every position
    if ((rc = attn_core_grads(c, L.attn, w + L.q, w + L.slotkv, oj, (int)ldoj, lj, w + L.da, (int)d.hs, dqj, dkj,
                              dvj)))
      return rc;
    if (l2c > 0.0) {  // gradients of the rotated Q and K, taken back through the rotation
      HIP_TRY(launch_rope_inverse(dqj, d.BT, (int)d.Hd, (int)d.d, 0, d.T, d.C, (int)d.r, (int)d.D, l2c, c.s));
      HIP_TRY(launch_rope_inverse(dkj, d.BS, (int)d.Hkd, (int)d.d, d.S, d.T, d.C, (int)d.r, (int)d.D, l2c, c.s));
    }
  }
  return TSP_OK;
}

int tsp_kv_grad_reduce(const tsp_dims* dims, const float* const* dkv_parts, float* dkv_own, void* stream) {
  g_err.clear();
  Dims d;
  int rc = check_dims(dims, &d);
  if (rc) return rc;
  if (d.S == 0) return TSP_OK;
  if (d.D > kMaxFold) return fail(TSP_E_SHAPE, "fold %lld exceeds %d", (long long)d.D, kMaxFold);
  if (d.d % 4) return fail(TSP_E_SHAPE, "head_dim must be a multiple of 4");
  if ((rc = check_ptrs({dkv_own})) || (rc = check_shards((const void* const*)dkv_parts, d.D, "dkv_parts")))
    return rc;
  KvGradReduceArgs a;
  memset(&a, 0, sizeof a);
  for (int64_t q = 0; q < d.D; q++) a.part[q] = dkv_parts[q];
  a.own = dkv_own;
  a.S = d.S;
  a.T = d.T;
  a.chunk = d.C;
  a.batch = d.B;
  a.rank = (int)d.r;
  a.fold = (int)d.D;
  a.hkd = (int)d.Hkd;
  a.hd = (int)d.d;
  HIP_TRY(launch_kv_grad_reduce(a, (hipStream_t)stream));
  return TSP_OK;
}

int tsp_layer_shard_backward_finish(const tsp_dims* dims, const void* x, const void* g1, const void* const* w_attn,
                                    const void* dx1, const float* dq, const float* dkv_own, void* dx, float* dg1,
                                    float* const* dw_qkv, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  Dims d;
  int rc = check_dims(dims, &d);
  if (rc) return rc;
  if (d.S == 0) return TSP_OK;
  if ((rc = check_attn_bwd_dims(d))) return rc;
  if ((rc = check_ptrs({x, g1, dx1, dq, dkv_own, dx, dg1, ws})) || (rc = check_shards(w_attn, d.D, "w_attn")) ||
      (rc = check_shards((const void* const*)dw_qkv, d.D, "dw_qkv")))
    return rc;
  const LayerBwd2Ws L = layer_bwd2_ws(d);
  if (ws_bytes < L.end) return fail(TSP_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.end);
  Ctx c{&d, (char*)ws, (hipStream_t)stream, (hipStream_t)stream, false, nullptr, false};
  char* w = c.ws;
  const int64_t N = (int64_t)qkv_rows(d);
  float* dn = (float*)(w + L.dn);
  HIP_TRY(launch_rmsnorm(d.dt, x, g1, w + L.n1, d.BT, (int)d.h, d.eps, c.s));
  HIP_TRY(launch_transpose(d.dt, w + L.n1, w + L.n1t, d.BT, d.h, d.h, d.BT, c.s));
  const size_t own_block = 2 * (size_t)d.Hkd * d.BT * d.d;  // one shard's [dK | dV] of the rank's rows
  for (int64_t j = 0; j < d.D; j++) {
    const float* dkj = dkv_own + (size_t)j * own_block;
    const float* dvj = dkj + (size_t)d.Hkd * d.BT * d.d;
    HIP_TRY(launch_qkv_grad_pack(d.dt, dq + (size_t)j * d.Hd * d.BT * d.d, dkj, dvj, w + L.g, d.BT, (int)d.hs,
                                 (int)d.ks, (int)d.d, c.s));
    // dn1 (+)= [dQ | dK | dV] . [W_Q; W_K; W_V]^T (B operand: the shard's block transposed)
    HIP_TRY(launch_transpose(d.dt, w_attn[j], w + L.wt, N, d.h, d.h, N, c.s));
    if ((rc = plain_gemm(c, w + L.g, N, w + L.wt, N, d.BT, d.h, N, dn, d.h, j > 0))) return rc;
    // this rank's partial gradient of the shard's Q|K|V block: [dQ | dK | dV]^T n1
    HIP_TRY(launch_transpose(d.dt, w + L.g, w + L.gt, d.BT, N, N, d.BT, c.s));
    if ((rc = plain_gemm(c, w + L.gt, d.BT, w + L.n1t, d.BT, N, d.h, d.BT, dw_qkv[j], d.h, false))) return rc;
  }
  HIP_TRY(launch_fill32(dg1, 0u, (size_t)d.h * 4, c.s));
  // the gain's partial sums go to n1t, free once the last shard's GEMMs have read it
  HIP_TRY(launch_rmsnorm_bwd(d.dt, x, g1, dn, dx1, dx, (float*)(w + L.rs), dg1, (float*)(w + L.n1t), d.BT, (int)d.h,
                             d.eps, c.s));
  return TSP_OK;
}

int tsp_attn_core_backward(const tsp_dims* dims, const void* q, const void* kv, const void* dout, float* dq,
                           float* dk, float* dv, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  Dims d;
  int rc = check_dims(dims, &d);
  if (rc) return rc;
  if (d.S == 0) return TSP_OK;
  if ((rc = check_attn_bwd_dims(d))) return rc;
  if ((rc = check_ptrs({q, kv, dout, dq, dk, dv, ws}))) return rc;
  const AttnBwdWs L = attn_bwd_ws(d);
  if (ws_bytes < L.end) return fail(TSP_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.end);
  Ctx c{&d, (char*)ws, (hipStream_t)stream, (hipStream_t)stream, false, nullptr, false};
  // forward recomputation: the group's output and each row's log-sum-exp
  if ((rc = attn_recompute(c, L, q, kv))) return rc;
  return attn_core_grads(c, L, q, kv, c.ws + L.o, (int)d.hs, (const float*)(c.ws + L.lse), dout, (int)d.hs, dq,
                         dk, dv);
}

int tsp_kv_shard(const tsp_dims* dims, const void* x, const void* g1, const void* const* w_attn,
                 void* kv, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  Dims d;
  int rc = check_dims(dims, &d);
  if (rc) return rc;
  if (d.S == 0) return TSP_OK;
  if ((rc = check_ptrs({x, g1, kv, ws})) || (rc = check_shards(w_attn, d.D, "w_attn"))) return rc;
  if (ws_bytes < kv_ws_bytes(d))
    return fail(TSP_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, kv_ws_bytes(d));
  Ctx c{&d, (char*)ws, (hipStream_t)stream, (hipStream_t)stream, false, nullptr,
        (d.flags & TSP_F_PROFILE) != 0};
  TIMED(c, TSP_K_RMSNORM, HIP_TRY(launch_rmsnorm(d.dt, x, g1, ws, d.BT, (int)d.h, d.eps, c.s)));
  const size_t kvbytes = kv_block_elems(d) * d.es;
  for (int64_t j = 0; j < d.D; j++) {
    TIMED(c, TSP_K_QKV,
          rc = qkv_gemm(c, ws, (const char*)w_attn[j], (int)d.hs, nullptr,
                        (char*)kv + (size_t)j * kvbytes));
    if (rc) return rc;
  }
  return TSP_OK;
}

int tsp_clock_probe(uint64_t* samples, int32_t n, int32_t interval_us, int32_t* wall_khz, void* stream) {
  g_err.clear();
  if (!samples || !wall_khz || n <= 0 || interval_us <= 0)
    return fail(TSP_E_INVAL, "clock probe needs a buffer, a wall-clock rate pointer, n > 0 and interval > 0");
  if (((uintptr_t)samples & 7) != 0) return fail(TSP_E_ALIGN, "samples must be 8-byte aligned");
  if ((int64_t)n * interval_us > 4000000)
    return fail(TSP_E_INVAL, "n * interval_us exceeds the probe's 4 s limit");
  int dev = 0, khz = 0;
  HIP_TRY(hipGetDevice(&dev));
  HIP_TRY(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev));
  if (khz <= 0) return fail(TSP_E_HIP, "device reports no wall-clock rate");
  *wall_khz = khz;
  const uint64_t ticks = (uint64_t)khz * (uint64_t)interval_us / 1000u;
  HIP_TRY(launch_clock_probe(samples, n, ticks ? ticks : 1, (hipStream_t)stream));
  return TSP_OK;
}

int tsp_profile_read(double* ms, int64_t* n, int reset) {
  g_err.clear();
  for (auto& p : g_prof.pending) {
    float t = 0.f;
    HIP_TRY(hipEventSynchronize(p.b));
    HIP_TRY(hipEventElapsedTime(&t, p.a, p.b));
    g_prof.ms[p.k] += t;
    g_prof.n[p.k] += 1;
    g_prof.pool.push_back(p.a);
    g_prof.pool.push_back(p.b);
  }
  g_prof.pending.clear();
  for (int k = 0; k < TSP_K_COUNT; k++) {
    if (ms) ms[k] = g_prof.ms[k];
    if (n) n[k] = g_prof.n[k];
    if (reset) {
      g_prof.ms[k] = 0;
      g_prof.n[k] = 0;
    }
  }
  return TSP_OK;
}

}  // extern "C"
