// Host side of the ring-attention step library: argument validation, the ring
// schedule, the double-buffered K/V rotation pipeline and the C ABI.
//
// Ring schedule (close-reading notes on "Ring Attention with Blockwise
// Transformers for Near-Infinite Context", §3.2 and the §3.5 walk-through):
// host r computes in round s with the block it holds, (r - s) mod D, while the
// block for round s+1 is in flight from the previous host.  On one GPU the
// "link" is an asynchronous device-to-device copy into one of two staging
// buffers on a library-owned side stream:
//
//   side:  copy(1)->buf1  copy(2)->buf0  [wait done1] copy(3)->buf1  [wait done2] copy(4)->buf0 ...
//   main:  kernel(0, own block)  [wait copied1] kernel(1, buf1)  [wait copied2] kernel(2, buf0) ...
//
// so the copy for round s+1 overlaps the kernel of round s, and a buffer is
// only refilled after the kernel that read it has finished (the resident
// "six blocks" of §3.4: Q, O, the K/V in use and the K/V in flight).  With a
// causal mask the rounds whose block lies in the future are dropped (every
// rank's own block comes first and is the masked diagonal).
//
// In the backward, the dK/dV and dQ kernels of a round read the same K/V
// block and write different outputs; with bf16 inputs the dK/dV kernel also
// writes the half copy of the block that the dQ kernel after it reads.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/ring_attn.h"
#include "kernels.h"
#include "ring_host.h"

namespace ra {

// ------------------------------------------------------------------ errors
static thread_local std::string g_last_error;

static int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

#define RA_HIP(call)                                                                  \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess)                                                             \
      return fail(RA_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(e_));         \
  } while (0)

// ------------------------------------------------------------------ schedule
std::vector<int> ring_schedule(int rank, int n_blocks, int causal) {
  std::vector<int> steps;
  for (int s = 0; s < n_blocks; ++s) {
    const int j = ((rank - s) % n_blocks + n_blocks) % n_blocks;
    if (causal && j > rank) continue;
    steps.push_back(j);
  }
  return steps;
}

// ------------------------------------------------------------------ validation (no HIP calls)
static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

int validate_common(const Shape& sh, const void* q, const void* const* kb, const void* const* vb) {
  if (!q) return fail(RA_ERR_INVALID_ARG, "q is NULL");
  if (!kb || !vb) return fail(RA_ERR_INVALID_ARG, "k_blocks/v_blocks array is NULL");
  if (sh.n_blocks < 1) return fail(RA_ERR_INVALID_ARG, "n_blocks must be >= 1 (got %d)", sh.n_blocks);
  if (sh.rank < 0 || sh.rank >= sh.n_blocks)
    return fail(RA_ERR_INVALID_ARG, "rank %d outside [0, %d)", sh.rank, sh.n_blocks);
  if (sh.block_len < 1) return fail(RA_ERR_INVALID_ARG, "block_len must be >= 1 (got %d)", sh.block_len);
  if (sh.heads < 1 || sh.kv_heads < 1)
    return fail(RA_ERR_INVALID_ARG, "heads and kv_heads must be >= 1 (got %d, %d)", sh.heads, sh.kv_heads);
  if (sh.heads % sh.kv_heads != 0)
    return fail(RA_ERR_INVALID_ARG, "heads (%d) must be a multiple of kv_heads (%d)", sh.heads, sh.kv_heads);
  if (sh.head_dim != 64 && sh.head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", sh.head_dim);
  const double elems = (double)sh.block_len * std::max(sh.heads, sh.kv_heads) * sh.head_dim;
  if (elems >= 2147483647.0)
    return fail(RA_ERR_INVALID_ARG, "block_len*heads*head_dim = %.0f exceeds 2^31-1", elems);
  for (int j = 0; j < sh.n_blocks; ++j)
    if (!kb[j] || !vb[j]) return fail(RA_ERR_INVALID_ARG, "k_blocks[%d] or v_blocks[%d] is NULL", j, j);
  if (sh.zigzag && sh.block_len % 2 != 0)
    return fail(RA_ERR_INVALID_ARG, "zig-zag layout needs an even block_len (got %d)", sh.block_len);
  return RA_OK;
}

int validate_outputs_disjoint(const Shape& sh, const void* q, const void* const* kb,
                              const void* const* vb, const void* const* outs, const size_t* out_bytes,
                              int n_outs, const char* const* names) {
  const size_t qb = sh.q_bytes(), kvb = sh.kv_bytes();
  for (int o = 0; o < n_outs; ++o) {
    if (!outs[o]) return fail(RA_ERR_INVALID_ARG, "%s is NULL", names[o]);
    if (overlaps(outs[o], out_bytes[o], q, qb)) return fail(RA_ERR_INVALID_ARG, "%s overlaps q", names[o]);
    for (int j = 0; j < sh.n_blocks; ++j)
      if (overlaps(outs[o], out_bytes[o], kb[j], kvb) || overlaps(outs[o], out_bytes[o], vb[j], kvb))
        return fail(RA_ERR_INVALID_ARG, "%s overlaps K/V block %d", names[o], j);
    for (int p = 0; p < o; ++p)
      if (overlaps(outs[o], out_bytes[o], outs[p], out_bytes[p]))
        return fail(RA_ERR_INVALID_ARG, "%s overlaps %s", names[o], names[p]);
  }
  return RA_OK;
}

// ------------------------------------------------------------------ per-device context
struct ProfRec {
  int kind;
  hipEvent_t a, b;
  int call;
};

struct Ctx {
  int device = -1;
  hipStream_t side = nullptr;
  hipEvent_t ev_entry = nullptr, ev_side_end = nullptr;
  hipEvent_t ev_copied[2] = {nullptr, nullptr}, ev_done[2] = {nullptr, nullptr};
  hipEvent_t ev_last = nullptr;  // end of the last call on this device (on that call's stream)
  bool last_valid = false;
  void* stage = nullptr;  // [kbuf0 | kbuf1 | vbuf0 | vbuf1]
  size_t stage_cap = 0;
  bool stage_owned = true;  // false: caller memory from ring_attn_set_workspace
  // backward workspace: row terms [delta | lse2] (fp32), then for bf16 inputs
  // the half copies [q16 | do16] of the query block and [k16 | v16] of one K/V block
  void* bwd = nullptr;
  size_t bwd_cap = 0;
  float* dec = nullptr;  // decode partials
  size_t dec_cap = 0;
  void* ffn = nullptr;   // blockwise feedforward intermediate (one row chunk)
  size_t ffn_cap = 0;
};

static std::mutex g_mu;
static std::vector<Ctx*> g_ctx;
static bool g_prof = false;
static std::vector<ProfRec> g_prof_recs;
static std::vector<hipEvent_t> g_prof_pool;
static int g_prof_call = 0;

static int get_ctx(Ctx** out) {
  int dev = 0;
  RA_HIP(hipGetDevice(&dev));
  for (Ctx* c : g_ctx)
    if (c->device == dev) {
      *out = c;
      return RA_OK;
    }
  Ctx* c = new Ctx();
  c->device = dev;
  hipError_t e = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking);
  hipEvent_t* evs[] = {&c->ev_entry, &c->ev_side_end, &c->ev_copied[0], &c->ev_copied[1], &c->ev_done[0],
                       &c->ev_done[1],  &c->ev_last};
  for (hipEvent_t* ev : evs)
    if (e == hipSuccess) e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
  if (e != hipSuccess) {
    delete c;
    return fail(RA_ERR_HIP, "creating side stream/events: %s", hipGetErrorString(e));
  }
  g_ctx.push_back(c);
  *out = c;
  return RA_OK;
}

// Calls on one device share its staging and workspace buffers, so they run one
// after another on the GPU even when issued on different streams: a call's
// stream first waits for the end of the previous call (an event recorded on
// that call's stream), and the call records its own end when it is done
// enqueueing.  Enqueueing itself is serialised by the library mutex.
struct CallOrder {
  Ctx* c;
  hipStream_t st;
  CallOrder(Ctx* c_, hipStream_t s) : c(c_), st(s) {}
  int begin() {
    if (c->last_valid) RA_HIP(hipStreamWaitEvent(st, c->ev_last, 0));
    return RA_OK;
  }
  ~CallOrder() {
    if (c && hipEventRecord(c->ev_last, st) == hipSuccess) c->last_valid = true;
  }
};

static int ensure_stage(Ctx* c, size_t bytes) {
  if (c->stage_cap >= bytes) return RA_OK;
  if (!c->stage_owned)
    return fail(RA_ERR_INVALID_ARG, "caller workspace holds %zu bytes, this call needs %zu", c->stage_cap,
                bytes);
  if (c->stage) {
    RA_HIP(hipDeviceSynchronize());
    RA_HIP(hipFree(c->stage));
    c->stage = nullptr;
    c->stage_cap = 0;
  }
  if (hipMalloc(&c->stage, bytes) != hipSuccess) {
    (void)hipGetLastError();
    c->stage = nullptr;
    return fail(RA_ERR_OOM, "could not allocate %zu bytes of K/V staging", bytes);
  }
  c->stage_cap = bytes;
  return RA_OK;
}

static int ensure_bwd(Ctx* c, size_t bytes) {
  if (c->bwd_cap >= bytes) return RA_OK;
  if (c->bwd) {
    RA_HIP(hipDeviceSynchronize());
    RA_HIP(hipFree(c->bwd));
    c->bwd = nullptr;
    c->bwd_cap = 0;
  }
  if (hipMalloc(&c->bwd, bytes) != hipSuccess) {
    (void)hipGetLastError();
    c->bwd = nullptr;
    return fail(RA_ERR_OOM, "could not allocate %zu bytes of backward workspace", bytes);
  }
  c->bwd_cap = bytes;
  return RA_OK;
}

// Regions of the backward workspace, each starting on a 256-byte boundary.
struct BwdLayout {
  size_t delta, lse2, q16, do16, k16, v16, total;
  explicit BwdLayout(const Shape& sh) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    delta = 0;
    lse2 = up(sh.lse_bytes());
    q16 = lse2 + up(sh.lse_bytes());
    if (sh.elem_bytes == 2) {  // half copies: 2 bytes per element, the inputs' own layouts
      do16 = q16 + up(sh.q_bytes());
      k16 = do16 + up(sh.q_bytes());
      v16 = k16 + up(sh.kv_bytes());
      total = v16 + up(sh.kv_bytes());
    } else {
      do16 = k16 = v16 = total = q16;
    }
  }
};

static int ensure_dec(Ctx* c, size_t bytes) {
  if (c->dec_cap >= bytes) return RA_OK;
  if (c->dec) {
    RA_HIP(hipDeviceSynchronize());
    RA_HIP(hipFree(c->dec));
    c->dec = nullptr;
    c->dec_cap = 0;
  }
  if (hipMalloc((void**)&c->dec, bytes) != hipSuccess) {
    (void)hipGetLastError();
    c->dec = nullptr;
    return fail(RA_ERR_OOM, "could not allocate %zu bytes for decode partials", bytes);
  }
  c->dec_cap = bytes;
  return RA_OK;
}

static int ensure_ffn(Ctx* c, size_t bytes) {
  if (c->ffn_cap >= bytes) return RA_OK;
  if (c->ffn) {
    RA_HIP(hipDeviceSynchronize());
    RA_HIP(hipFree(c->ffn));
    c->ffn = nullptr;
    c->ffn_cap = 0;
  }
  if (hipMalloc(&c->ffn, bytes) != hipSuccess) {
    (void)hipGetLastError();
    c->ffn = nullptr;
    return fail(RA_ERR_OOM, "could not allocate %zu bytes for the feedforward intermediate", bytes);
  }
  c->ffn_cap = bytes;
  return RA_OK;
}

// profiling helpers (only active while enabled)
static hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

struct ProfScope {
  int kind;
  hipStream_t st;
  hipEvent_t a = nullptr;
  ProfScope(int k, hipStream_t s) : kind(k), st(s) {
    if (g_prof) {
      a = prof_event();
      if (a) (void)hipEventRecord(a, st);
    }
  }
  ~ProfScope() {
    if (a) {
      hipEvent_t b = prof_event();
      if (b) {
        (void)hipEventRecord(b, st);
        g_prof_recs.push_back(ProfRec{kind, a, b, g_prof_call});
      }
    }
  }
};

enum {
  KIND_FWD = 0,
  KIND_DKDV = 1,
  KIND_DQ = 2,
  KIND_PRE = 3,
  KIND_MERGE = 4,
  KIND_COPY = 5,
  KIND_DEC_PART = 6,
  KIND_DEC_MERGE = 7,
  KIND_FFN_UP = 8,
  KIND_FFN_DOWN = 9,
  KIND_COUNT = 10
};

// ------------------------------------------------------------------ copy engine choice
static hipMemcpyKind copy_kind() {
  static int kind = -1;
  if (kind < 0) {
    const char* s = getenv("RING_ATTN_COPY");
    kind = (s && strcmp(s, "kernel") == 0) ? 1 : 0;
  }
  return kind == 1 ? hipMemcpyDeviceToDevice : hipMemcpyDeviceToDeviceNoCU;
}

static int g_poison = 0;
static long long g_delay_cycles = 0;

static bool log_schedule() {
  static int v = -1;
  if (v < 0) {
    const char* s = getenv("RING_ATTN_LOG");
    v = (s && s[0] == '1') ? 1 : 0;
  }
  return v == 1;
}

// ------------------------------------------------------------------ the ring pipeline
// step_fn(s, j, k_ptr, v_ptr) launches round s's kernels on `stream`.
template <typename StepFn>
static int run_ring(Ctx* c, const Shape& sh, const void* const* kb, const void* const* vb,
                    hipStream_t stream, StepFn&& step_fn) {
  const std::vector<int> steps = ring_schedule(sh.rank, sh.n_blocks, sh.schedule_causal());
  const int S = (int)steps.size();
  const size_t kvb = sh.kv_bytes();
  if (log_schedule()) {
    fprintf(stderr, "[ring_attn] rank %d/%d causal=%d rounds:", sh.rank, sh.n_blocks, sh.causal);
    for (int j : steps) fprintf(stderr, " %d", j);
    fprintf(stderr, "\n");
  }
  char* kbuf[2] = {nullptr, nullptr};
  char* vbuf[2] = {nullptr, nullptr};
  if (S > 1) {
    int st = ensure_stage(c, 4 * kvb);
    if (st != RA_OK) return st;
    char* base = static_cast<char*>(c->stage);
    kbuf[0] = base;
    kbuf[1] = base + kvb;
    vbuf[0] = base + 2 * kvb;
    vbuf[1] = base + 3 * kvb;
    RA_HIP(hipEventRecord(c->ev_entry, stream));
    RA_HIP(hipStreamWaitEvent(c->side, c->ev_entry, 0));
  }
  auto issue_copy = [&](int s) -> int {
    const int b = s & 1, j = steps[s];
    if (g_poison && s >= 3) RA_HIP(launch_fill_nan(kbuf[b], vbuf[b], kvb, c->side));
    if (g_delay_cycles > 0) RA_HIP(launch_spin(g_delay_cycles, c->side));
    {
      ProfScope ps(KIND_COPY, c->side);
      RA_HIP(hipMemcpyAsync(kbuf[b], kb[j], kvb, copy_kind(), c->side));
      RA_HIP(hipMemcpyAsync(vbuf[b], vb[j], kvb, copy_kind(), c->side));
    }
    RA_HIP(hipEventRecord(c->ev_copied[b], c->side));
    return RA_OK;
  };
  int st;
  if (S > 1 && (st = issue_copy(1)) != RA_OK) return st;
  if (S > 2 && (st = issue_copy(2)) != RA_OK) return st;
  if ((st = step_fn(0, steps[0], kb[steps[0]], vb[steps[0]])) != RA_OK) return st;
  for (int s = 1; s < S; ++s) {
    const int b = s & 1;
    RA_HIP(hipStreamWaitEvent(stream, c->ev_copied[b], 0));
    if ((st = step_fn(s, steps[s], kbuf[b], vbuf[b])) != RA_OK) return st;
    if (s + 2 < S) {
      RA_HIP(hipEventRecord(c->ev_done[b], stream));
      RA_HIP(hipStreamWaitEvent(c->side, c->ev_done[b], 0));
      if ((st = issue_copy(s + 2)) != RA_OK) return st;
    }
  }
  if (S > 1) {
    RA_HIP(hipEventRecord(c->ev_side_end, c->side));
    RA_HIP(hipStreamWaitEvent(stream, c->ev_side_end, 0));
  }
  return RA_OK;
}

static float rsqrt_dim(int d) { return 1.0f / std::sqrt((float)d); }

// Zig-zag layout: block b holds sequence chunks b (first half) and 2D-1-b
// (second half), so every rank's causal work is the same.
static int zz_chunk(int block, int half, int n_blocks) { return half == 0 ? block : 2 * n_blocks - 1 - block; }

// The (query half, key half) chunk pairs of one zig-zag round, grouped into
// kernel sub-problems.  `own` is the side whose rows a sub-problem writes (the
// query half for the forward and dQ, the key half for dK/dV), `other` the
// side it streams.  When one `own` half sees both `other` halves and neither
// pair is a causal diagonal, the two pairs become one sub-problem over the
// whole other block (contiguous in memory), so a workgroup streams a
// full-length block as in the contiguous layout.  The sub-problems are then
// paired into launches: two per launch when they write different halves and
// have the same lengths.
struct ZzSpan {
  int own, other0, n_other;  // n_other 2: both other halves, from half 0
  bool diag;
};
struct ZzLaunch {
  ZzSpan sub[2];
  int nsub;
};
static std::vector<ZzLaunch> zz_launches(const Shape& sh, int j, bool own_is_query) {
  std::vector<ZzSpan> sp[2];
  for (int o = 0; o < 2; ++o) {
    bool live[2], diag[2];
    for (int t = 0; t < 2; ++t) {
      const int u = own_is_query ? o : t, v = own_is_query ? t : o;  // query half u, key half v
      const int qc = zz_chunk(sh.rank, u, sh.n_blocks), kc = zz_chunk(j, v, sh.n_blocks);
      live[t] = !(sh.causal && kc > qc);  // a chunk wholly in the queries' future is skipped
      diag[t] = sh.causal && kc == qc;
    }
    if (live[0] && live[1] && !diag[0] && !diag[1]) {
      sp[o].push_back({o, 0, 2, false});
    } else {
      for (int t = 0; t < 2; ++t)
        if (live[t]) sp[o].push_back({o, t, 1, diag[t]});
    }
  }
  std::vector<ZzLaunch> out;
  size_t i0 = 0, i1 = 0;
  while (i0 < sp[0].size() || i1 < sp[1].size()) {
    ZzLaunch l{};
    if (i0 < sp[0].size()) {
      l.sub[l.nsub++] = sp[0][i0++];
      if (i1 < sp[1].size() && sp[1][i1].n_other == l.sub[0].n_other) l.sub[l.nsub++] = sp[1][i1++];
    } else {
      l.sub[l.nsub++] = sp[1][i1++];
    }
    out.push_back(l);
  }
  return out;
}

// Query heads that share one workgroup: the largest common divisor of the group
// size and the wave count (each wave owns 32 rows of one head).
static int heads_per_block(int group, int waves) {
  for (int x = waves; x >= 1; --x)
    if (group % x == 0 && waves % x == 0) return x;
  return 1;
}

int fwd_impl(const void* q, const void* const* kb, const void* const* vb, const Shape& sh, float* out,
             float* lse, hipStream_t stream) {
  int st = validate_common(sh, q, kb, vb);
  if (st != RA_OK) return st;
  const void* outs[] = {out, lse};
  const size_t ob[] = {sh.out_bytes(), sh.lse_bytes()};
  const char* names[] = {"out", "lse"};
  if ((st = validate_outputs_disjoint(sh, q, kb, vb, outs, ob, 2, names)) != RA_OK) return st;

  std::lock_guard<std::mutex> lk(g_mu);
  Ctx* c = nullptr;
  if ((st = get_ctx(&c)) != RA_OK) return st;
  CallOrder order(c, stream);
  if ((st = order.begin()) != RA_OK) return st;
  ++g_prof_call;
  const int group = sh.heads / sh.kv_heads;
  const int hpw = heads_per_block(group, fwd_waves_per_block(sh.elem_bytes));
  FwdArgs base{};
  base.q = q;
  base.out = out;
  base.lse = lse;
  base.len = sh.block_len;
  base.klen = sh.block_len;
  base.ls = sh.block_len;
  base.hq = sh.heads;
  base.hkv = sh.kv_heads;
  base.group = group;
  base.hpw = hpw;
  base.hsub = group / hpw;
  base.scale_log2 = 1.4426950408889634f * rsqrt_dim(sh.head_dim);
  bool first_half[2] = {true, true};
  auto step = [&](int s, int j, const void* kp, const void* vp) -> int {
    if (!sh.zigzag) {
      FwdArgs a = base;
      a.k = kp;
      a.v = vp;
      a.diag = (sh.causal && j == sh.rank) ? 1 : 0;
      a.first = (s == 0) ? 1 : 0;
      ProfScope ps(KIND_FWD, stream);
      RA_HIP(launch_fwd_step(&a, 1, sh.elem_bytes, sh.head_dim, stream));
      return RA_OK;
    }
    // zig-zag: query half u holds chunk zz_chunk(rank, u), key half v chunk zz_chunk(j, v).
    // Sub-problems of one launch write different query halves; those of one query half
    // follow one another (the later ones merge into the earlier's output).
    const int h = sh.block_len / 2;
    for (const ZzLaunch& l : zz_launches(sh, j, true)) {
      FwdArgs sub[2];
      for (int i = 0; i < l.nsub; ++i) {
        const ZzSpan& z = l.sub[i];
        FwdArgs& a = sub[i];
        a = base;
        a.q = static_cast<const char*>(q) + (size_t)z.own * h * sh.heads * sh.head_dim * sh.elem_bytes;
        a.out = out + (size_t)z.own * h * sh.heads * sh.head_dim;
        a.lse = lse + (size_t)z.own * h;
        a.k = static_cast<const char*>(kp) + (size_t)z.other0 * h * sh.kv_heads * sh.head_dim * sh.elem_bytes;
        a.v = static_cast<const char*>(vp) + (size_t)z.other0 * h * sh.kv_heads * sh.head_dim * sh.elem_bytes;
        a.len = h;
        a.klen = z.n_other * h;
        a.diag = z.diag ? 1 : 0;
        a.first = first_half[z.own] ? 1 : 0;
        first_half[z.own] = false;
      }
      ProfScope ps(KIND_FWD, stream);
      RA_HIP(launch_fwd_step(sub, l.nsub, sh.elem_bytes, sh.head_dim, stream));
    }
    return RA_OK;
  };
  return run_ring(c, sh, kb, vb, stream, step);
}

int bwd_impl(const void* q, const void* const* kb, const void* const* vb, const float* out,
             const void* dout, const float* lse, const Shape& sh, float* dq, float* const* dkb,
             float* const* dvb, hipStream_t stream) {
  int st = validate_common(sh, q, kb, vb);
  if (st != RA_OK) return st;
  if (!out || !dout || !lse) return fail(RA_ERR_INVALID_ARG, "out, dout or lse is NULL");
  if (!dkb || !dvb) return fail(RA_ERR_INVALID_ARG, "dk_blocks/dv_blocks array is NULL");
  std::vector<const void*> outs;
  std::vector<size_t> ob;
  std::vector<std::string> nm;
  outs.push_back(dq);
  ob.push_back(sh.out_bytes());
  nm.push_back("dq");
  for (int j = 0; j < sh.n_blocks; ++j) {
    outs.push_back(dkb[j]);
    ob.push_back(sh.kv_f32_bytes());
    nm.push_back("dk_blocks[" + std::to_string(j) + "]");
    outs.push_back(dvb[j]);
    ob.push_back(sh.kv_f32_bytes());
    nm.push_back("dv_blocks[" + std::to_string(j) + "]");
  }
  // gradients must also stay clear of the other read-only inputs
  const void* ro[] = {out, dout, lse};
  const size_t rob[] = {sh.out_bytes(), sh.q_bytes(), sh.lse_bytes()};
  std::vector<const char*> names;
  for (auto& s : nm) names.push_back(s.c_str());
  if ((st = validate_outputs_disjoint(sh, q, kb, vb, outs.data(), ob.data(), (int)outs.size(),
                                      names.data())) != RA_OK)
    return st;
  for (size_t o = 0; o < outs.size(); ++o)
    for (int r = 0; r < 3; ++r)
      if (overlaps(outs[o], ob[o], ro[r], rob[r]))
        return fail(RA_ERR_INVALID_ARG, "%s overlaps a forward input (out/dout/lse)", names[o]);

  std::lock_guard<std::mutex> lk(g_mu);
  Ctx* c = nullptr;
  if ((st = get_ctx(&c)) != RA_OK) return st;
  CallOrder order(c, stream);
  if ((st = order.begin()) != RA_OK) return st;
  ++g_prof_call;
  // staging first: a caller workspace that is too small must fail before anything is enqueued
  if (ring_schedule(sh.rank, sh.n_blocks, sh.schedule_causal()).size() > 1 &&
      (st = ensure_stage(c, 4 * sh.kv_bytes())) != RA_OK)
    return st;
  const BwdLayout L(sh);
  if ((st = ensure_bwd(c, L.total)) != RA_OK) return st;
  char* ws = static_cast<char*>(c->bwd);
  float* delta = reinterpret_cast<float*>(ws + L.delta);
  float* lse2 = reinterpret_cast<float*>(ws + L.lse2);
  const bool half = sh.elem_bytes == 2;  // bf16 inputs: the kernels contract half copies
  void* q16 = half ? ws + L.q16 : nullptr;
  void* do16 = half ? ws + L.do16 : nullptr;
  char* k16 = half ? ws + L.k16 : nullptr;
  char* v16 = half ? ws + L.v16 : nullptr;
  {
    BwdPreArgs p{dout, out, lse, delta, lse2, sh.block_len, sh.heads, sh.block_len, q, q16, do16};
    ProfScope ps(KIND_PRE, stream);
    RA_HIP(launch_bwd_pre(p, sh.elem_bytes, sh.head_dim, stream));
  }
  const void* qk = half ? q16 : q;      // what the kernels read as q and dout
  const void* dok = half ? do16 : dout;
  const float scale = rsqrt_dim(sh.head_dim);
  const int group = sh.heads / sh.kv_heads;
  const int hpw =
      heads_per_block(group, sh.elem_bytes == 2 ? bwd_bf16_waves_per_block() : bwd_dq_waves_per_block());
  BwdArgs base{};
  base.q = qk;
  base.dout = dok;
  base.lse = lse;
  base.delta = delta;
  base.lse2 = lse2;
  base.dq = dq;
  base.len = sh.block_len;
  base.klen = sh.block_len;
  base.ls = sh.block_len;
  base.hq = sh.heads;
  base.hkv = sh.kv_heads;
  base.group = group;
  base.hpw = hpw;
  base.hsub = group / hpw;
  base.scale = scale;
  base.scale_log2 = 1.4426950408889634f * scale;
  auto launch_dkdv = [&](const BwdArgs* a, int nsub) -> int {
    ProfScope ps(KIND_DKDV, stream);
    RA_HIP(launch_bwd_dkdv(a, nsub, sh.elem_bytes, sh.head_dim, stream));
    return RA_OK;
  };
  auto launch_dq = [&](const BwdArgs* a, int nsub) -> int {
    ProfScope ps(KIND_DQ, stream);
    RA_HIP(launch_bwd_dq(a, nsub, sh.elem_bytes, sh.head_dim, stream));
    return RA_OK;
  };
  // bf16: the dQ kernel reads the half copy of the block that the dK/dV kernel wrote
  auto for_dq = [&](BwdArgs a) {
    if (half) {
      a.k = a.k16;
      a.v = a.v16;
    }
    return a;
  };
  bool first_half[2] = {true, true};
  auto bwd_round = [&](int s, int j, const void* kp, const void* vp) -> int {
    if (!sh.zigzag) {
      BwdArgs a = base;
      a.k = kp;
      a.v = vp;
      a.k16 = k16;
      a.v16 = v16;
      a.dk = dkb[j];
      a.dv = dvb[j];
      a.diag = (sh.causal && j == sh.rank) ? 1 : 0;
      a.first = (s == 0) ? 1 : 0;
      int st2 = launch_dkdv(&a, 1);
      if (st2 != RA_OK) return st2;
      const BwdArgs b = for_dq(a);
      return launch_dq(&b, 1);
    }
    // zig-zag: query half u holds chunk zz_chunk(rank, u), key half v chunk zz_chunk(j, v).
    // dK/dV sub-problems of one launch write different key halves, dQ sub-problems
    // different query halves.  Every live key half is covered by some dK/dV launch, which
    // writes its half copy before the dQ launches of the round read it.
    const int h = sh.block_len / 2;
    const size_t qrow = (size_t)sh.heads * sh.head_dim, krow = (size_t)sh.kv_heads * sh.head_dim;
    // query halves [u0, u0 + nu) against key halves [v0, v0 + nv)
    auto args = [&](int u0, int nu, int v0, int nv, bool diag) {
      BwdArgs a = base;
      a.q = static_cast<const char*>(qk) + u0 * h * qrow * sh.elem_bytes;
      a.dout = static_cast<const char*>(dok) + u0 * h * qrow * sh.elem_bytes;
      a.lse = lse + (size_t)u0 * h;
      a.delta = delta + (size_t)u0 * h;
      a.lse2 = lse2 + (size_t)u0 * h;
      a.dq = dq + u0 * h * qrow;
      a.k = static_cast<const char*>(kp) + v0 * h * krow * sh.elem_bytes;
      a.v = static_cast<const char*>(vp) + v0 * h * krow * sh.elem_bytes;
      a.k16 = half ? k16 + v0 * h * krow * 2 : nullptr;
      a.v16 = half ? v16 + v0 * h * krow * 2 : nullptr;
      a.dk = dkb[j] + v0 * h * krow;
      a.dv = dvb[j] + v0 * h * krow;
      a.len = nu * h;
      a.klen = nv * h;
      a.diag = diag ? 1 : 0;
      return a;
    };
    for (const ZzLaunch& l : zz_launches(sh, j, false)) {  // own = key half
      BwdArgs sub[2];
      for (int i = 0; i < l.nsub; ++i) {
        const ZzSpan& z = l.sub[i];
        sub[i] = args(z.other0, z.n_other, z.own, 1, z.diag);
      }
      int st2 = launch_dkdv(sub, l.nsub);
      if (st2 != RA_OK) return st2;
    }
    for (const ZzLaunch& l : zz_launches(sh, j, true)) {  // own = query half
      BwdArgs sub[2];
      for (int i = 0; i < l.nsub; ++i) {
        const ZzSpan& z = l.sub[i];
        sub[i] = for_dq(args(z.own, 1, z.other0, z.n_other, z.diag));
        sub[i].first = first_half[z.own] ? 1 : 0;  // dQ rows of half u: written by the first, then accumulated
        first_half[z.own] = false;
      }
      int st2 = launch_dq(sub, l.nsub);
      if (st2 != RA_OK) return st2;
    }
    return RA_OK;
  };
  return run_ring(c, sh, kb, vb, stream, bwd_round);
}

int merge_impl(const float* oa, const float* la, const float* obp, const float* lb, int rows, int heads,
               int head_dim, float* out, float* lse, hipStream_t stream) {
  if (!oa || !la || !obp || !lb || !out || !lse)
    return fail(RA_ERR_INVALID_ARG, "merge: NULL pointer argument");
  if (rows < 0 || heads < 1 || head_dim < 1)
    return fail(RA_ERR_INVALID_ARG, "merge: bad sizes rows=%d heads=%d head_dim=%d", rows, heads, head_dim);
  if ((double)rows * heads * head_dim >= 2147483647.0)
    return fail(RA_ERR_INVALID_ARG, "merge: rows*heads*head_dim exceeds 2^31-1");
  const size_t obytes = (size_t)rows * heads * head_dim * 4, lbytes = (size_t)rows * heads * 4;
  // exact aliasing with an input is the supported in-place form; partial overlap is not
  const void* ins_o[] = {oa, obp};
  const void* ins_l[] = {la, lb};
  for (int i = 0; i < 2; ++i) {
    if (out != ins_o[i] && overlaps(out, obytes, ins_o[i], obytes))
      return fail(RA_ERR_INVALID_ARG, "merge: out partially overlaps an input");
    if (lse != ins_l[i] && overlaps(lse, lbytes, ins_l[i], lbytes))
      return fail(RA_ERR_INVALID_ARG, "merge: lse partially overlaps an input");
    if (overlaps(out, obytes, ins_l[i], lbytes) || overlaps(lse, lbytes, ins_o[i], obytes))
      return fail(RA_ERR_INVALID_ARG, "merge: out/lse overlap the other kind of input");
  }
  if (overlaps(out, obytes, lse, lbytes)) return fail(RA_ERR_INVALID_ARG, "merge: out overlaps lse");
  if (rows == 0) return RA_OK;
  std::lock_guard<std::mutex> lk(g_mu);
  ++g_prof_call;
  MergeArgs a{oa, la, obp, lb, out, lse, rows, heads, head_dim};
  ProfScope ps(KIND_MERGE, stream);
  RA_HIP(launch_merge(a, stream));
  return RA_OK;
}

// ------------------------------------------------------------------ profiling readout
int debug_set(int poison, long long delay_cycles) {
  if (delay_cycles < 0) return fail(RA_ERR_INVALID_ARG, "delay_cycles must be >= 0");
  std::lock_guard<std::mutex> lk(g_mu);
  g_poison = poison != 0;
  g_delay_cycles = delay_cycles;
  return RA_OK;
}

int profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_prof = on != 0;
  return RA_OK;
}

int profile_read(double* ms, int* count, double* copy_ms, double* hidden_ms) {
  if (!ms || !count) return fail(RA_ERR_INVALID_ARG, "profile_read: NULL output array");
  std::lock_guard<std::mutex> lk(g_mu);
  for (int k = 0; k < KIND_COUNT; ++k) {
    ms[k] = 0.0;
    count[k] = 0;
  }
  double cms = 0.0, hid = 0.0;
  if (!g_prof_recs.empty()) {
    hipEvent_t ref = g_prof_recs.front().a;
    for (auto& r : g_prof_recs) RA_HIP(hipEventSynchronize(r.b));
    struct Iv {
      double a, b;
      int call;
    };
    std::vector<Iv> kern, copy;
    for (auto& r : g_prof_recs) {
      float ta = 0.f, tb = 0.f;
      RA_HIP(hipEventElapsedTime(&ta, ref, r.a));
      RA_HIP(hipEventElapsedTime(&tb, ref, r.b));
      ms[r.kind] += tb - ta;
      count[r.kind] += 1;
      if (r.kind == KIND_COPY) copy.push_back({ta, tb, r.call});
      else kern.push_back({ta, tb, r.call});
    }
    for (auto& cp : copy) {
      cms += cp.b - cp.a;
      // overlap of this copy with the union of the kernel intervals of the same call
      std::vector<std::pair<double, double>> cut;
      for (auto& k : kern) {
        if (k.call != cp.call) continue;
        const double lo = std::max(cp.a, k.a), hi = std::min(cp.b, k.b);
        if (hi > lo) cut.push_back({lo, hi});
      }
      std::sort(cut.begin(), cut.end());
      double cur_lo = -1e300, cur_hi = -1e300;
      for (auto& iv : cut) {
        if (iv.first > cur_hi) {
          if (cur_hi > cur_lo) hid += cur_hi - cur_lo;
          cur_lo = iv.first;
          cur_hi = iv.second;
        } else {
          cur_hi = std::max(cur_hi, iv.second);
        }
      }
      if (cur_hi > cur_lo) hid += cur_hi - cur_lo;
    }
    for (auto& r : g_prof_recs) {
      g_prof_pool.push_back(r.a);
      g_prof_pool.push_back(r.b);
    }
    g_prof_recs.clear();
  }
  if (copy_ms) *copy_ms = cms;
  if (hidden_ms) *hidden_ms = hid;
  return RA_OK;
}

#ifndef RA_DEC_WAVES
#define RA_DEC_WAVES 1024
#endif

// noalloc: the partials go to the library's fixed device array (decode_scratch)
// instead of the lazily grown per-device buffer; nothing is allocated, no
// library stream or event is created, and the call is not ordered against
// other calls (callers that overlap such calls on one GPU race on the array).
int decode_impl(const void* q, const void* const* kb, const void* const* vb, int n_blocks, int block_len,
                int q_len, int heads, int kv_heads, int head_dim, long long q_pos0, float* out, float* lse,
                hipStream_t stream, bool noalloc) {
  if (!q || !out || !lse) return fail(RA_ERR_INVALID_ARG, "q, out and lse must be non-NULL");
  if (!kb || !vb) return fail(RA_ERR_INVALID_ARG, "k_blocks/v_blocks array is NULL");
  if (n_blocks < 1 || n_blocks > kDecodeMaxBlocks)
    return fail(RA_ERR_INVALID_ARG, "n_blocks %d outside [1, %d]", n_blocks, kDecodeMaxBlocks);
  if (block_len < 1 || q_len < 1) return fail(RA_ERR_INVALID_ARG, "block_len and q_len must be >= 1");
  if (heads < 1 || kv_heads < 1 || heads % kv_heads != 0)
    return fail(RA_ERR_INVALID_ARG, "heads (%d) must be a positive multiple of kv_heads (%d)", heads, kv_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", head_dim);
  const int group = heads / kv_heads;
  if (group > 32)
    return fail(RA_ERR_UNSUPPORTED, "decode takes at most 32 query heads per K/V head (group %d)", group);
  // a pass holds at most 32 query rows per K/V head (group x rows of the pass); longer
  // query blocks run as successive passes over row chunks, each streaming the K/V again
  const int pass_rows = std::min(q_len, 32 / group);
  if (q_pos0 < 0) return fail(RA_ERR_INVALID_ARG, "q_pos0 must be >= 0");
  if ((double)block_len * kv_heads * head_dim >= 2147483647.0)
    return fail(RA_ERR_INVALID_ARG, "block_len*kv_heads*head_dim exceeds 2^31-1");
  for (int j = 0; j < n_blocks; ++j)
    if (!kb[j] || !vb[j]) return fail(RA_ERR_INVALID_ARG, "k_blocks[%d] or v_blocks[%d] is NULL", j, j);
  const size_t qbytes = (size_t)q_len * heads * head_dim * 2, obytes = (size_t)q_len * heads * head_dim * 4,
               lbytes = (size_t)heads * q_len * 4, kvb = (size_t)block_len * kv_heads * head_dim * 2;
  if (overlaps(out, obytes, lse, lbytes)) return fail(RA_ERR_INVALID_ARG, "out overlaps lse");
  const void* outs[2] = {out, lse};
  const size_t ob[2] = {obytes, lbytes};
  for (int o = 0; o < 2; ++o) {
    if (overlaps(outs[o], ob[o], q, qbytes)) return fail(RA_ERR_INVALID_ARG, "%s overlaps q", o ? "lse" : "out");
    for (int j = 0; j < n_blocks; ++j)
      if (overlaps(outs[o], ob[o], kb[j], kvb) || overlaps(outs[o], ob[o], vb[j], kvb))
        return fail(RA_ERR_INVALID_ARG, "%s overlaps K/V block %d", o ? "lse" : "out", j);
  }
  // keys per wave: about RA_DEC_WAVES waves over the whole context, rounded to a power of
  // two (so that power-of-two blocks split without a short last chunk), 256..8192 keys each
  const double total = (double)n_blocks * kv_heads * block_len;
  const double target = std::max(256.0, std::min(8192.0, total / (double)RA_DEC_WAVES));
  const int chunk = 1 << (int)std::lround(std::log2(target));
  const int n_chunks = (block_len + chunk - 1) / chunk;
  const int rows = group * pass_rows;
  const size_t n_parts = (size_t)n_blocks * n_chunks;
  const size_t need = (size_t)kv_heads * n_parts * rows * (head_dim + 1) * sizeof(float);

  std::lock_guard<std::mutex> lk(g_mu);
  float* part = nullptr;
  CallOrder order(nullptr, stream);  // ordered against other calls unless noalloc
  if (noalloc) {
    size_t cap = 0;
    RA_HIP(decode_scratch(&part, &cap));
    if (need > cap)
      return fail(RA_ERR_INVALID_ARG,
                  "decode partials need %zu bytes; the fixed scratch of the no-allocation entry point holds %zu",
                  need, cap);
  } else {
    Ctx* c = nullptr;
    int st = get_ctx(&c);
    if (st != RA_OK) return st;
    order.c = c;
    if ((st = order.begin()) != RA_OK) return st;
    if ((st = ensure_dec(c, need)) != RA_OK) return st;
    part = c->dec;
  }
  DecodeArgs a{};
  a.q = q;
  for (int j = 0; j < n_blocks; ++j) {
    a.kblk[j] = kb[j];
    a.vblk[j] = vb[j];
  }
  a.out = out;
  a.lse = lse;
  a.part_o = part;
  a.part_lse = part + (size_t)kv_heads * n_parts * rows * head_dim;
  a.q_pos0 = q_pos0;
  a.n_blocks = n_blocks;
  a.len = block_len;
  a.q_len = q_len;
  a.hq = heads;
  a.hkv = kv_heads;
  a.group = group;
  a.chunk = chunk;
  a.n_chunks = n_chunks;
  a.n_parts = (int)n_parts;
  a.scale_log2 = 1.4426950408889634f * rsqrt_dim(head_dim);
  a.ls = q_len;
  ++g_prof_call;
  for (int r0 = 0; r0 < q_len; r0 += pass_rows) {  // the passes share the partials buffer in stream order
    a.q = static_cast<const char*>(q) + (size_t)r0 * heads * head_dim * 2;
    a.out = out + (size_t)r0 * heads * head_dim;
    a.lse = lse + r0;
    a.q_pos0 = q_pos0 + r0;
    a.q_len = std::min(pass_rows, q_len - r0);
    {
      ProfScope ps(KIND_DEC_PART, stream);
      RA_HIP(launch_decode_partial(a, head_dim, stream));
    }
    {
      ProfScope ps(KIND_DEC_MERGE, stream);
      RA_HIP(launch_decode_merge(a, head_dim, stream));
    }
  }
  return RA_OK;
}

int ffn_impl(const void* x, const void* w1, const float* b1, const void* w2, const float* b2, int rows, int hidden,
             int ffn, int chunk_rows, float* y, hipStream_t stream) {
  if (!x || !w1 || !w2 || !y) return fail(RA_ERR_INVALID_ARG, "x, w1, w2 and y must be non-NULL");
  if (rows < 1) return fail(RA_ERR_INVALID_ARG, "rows must be >= 1 (got %d)", rows);
  const int tn = gemm_tile_n();
  if (hidden < tn || ffn < tn || hidden % tn != 0 || ffn % tn != 0)
    return fail(RA_ERR_UNSUPPORTED, "hidden (%d) and ffn (%d) must be positive multiples of %d", hidden, ffn, tn);
  if (chunk_rows < 0) return fail(RA_ERR_INVALID_ARG, "chunk_rows must be >= 0 (0: all rows at once)");
  const int chunk = (chunk_rows == 0 || chunk_rows > rows) ? rows : chunk_rows;
  // byte offsets inside one operand are 32-bit in the kernel
  const double lim = 4294967295.0;
  if ((double)rows * hidden * 4 >= lim || (double)chunk * ffn * 2 >= lim || (double)ffn * hidden * 2 >= lim)
    return fail(RA_ERR_INVALID_ARG, "operand larger than 4 GiB (rows %d, hidden %d, ffn %d)", rows, hidden, ffn);
  const size_t xb = (size_t)rows * hidden * 2, yb = (size_t)rows * hidden * 4, wb = (size_t)ffn * hidden * 2;
  const void* ins[] = {x, w1, w2, b1, b2};
  const size_t inb[] = {xb, wb, wb, (size_t)ffn * 4, (size_t)hidden * 4};
  for (int i = 0; i < 5; ++i)
    if (ins[i] && overlaps(y, yb, ins[i], inb[i])) return fail(RA_ERR_INVALID_ARG, "y overlaps an input");

  std::lock_guard<std::mutex> lk(g_mu);
  Ctx* c = nullptr;
  int st = get_ctx(&c);
  if (st != RA_OK) return st;
  CallOrder order(c, stream);
  if ((st = order.begin()) != RA_OK) return st;
  if ((st = ensure_ffn(c, (size_t)chunk * ffn * 2)) != RA_OK) return st;
  ++g_prof_call;
  for (int r0 = 0; r0 < rows; r0 += chunk) {
    const int m = std::min(chunk, rows - r0);
    GemmArgs up{static_cast<const char*>(x) + (size_t)r0 * hidden * 2, w1, c->ffn, b1, m, ffn, hidden, hidden, hidden,
                ffn};
    {
      ProfScope ps(KIND_FFN_UP, stream);
      RA_HIP(launch_gemm_bt(up, true, stream));
    }
    GemmArgs down{c->ffn, w2, y + (size_t)r0 * hidden, b2, m, hidden, ffn, ffn, ffn, hidden};
    {
      ProfScope ps(KIND_FFN_DOWN, stream);
      RA_HIP(launch_gemm_bt(down, false, stream));
    }
  }
  return RA_OK;
}

int set_workspace(void* ptr, size_t bytes) {
  if ((ptr == nullptr) != (bytes == 0))
    return fail(RA_ERR_INVALID_ARG, "workspace pointer and size must be both set or both zero");
  if ((uintptr_t)ptr % 256 != 0) return fail(RA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  std::lock_guard<std::mutex> lk(g_mu);
  Ctx* c = nullptr;
  int st = get_ctx(&c);
  if (st != RA_OK) return st;
  // every call that may still read or fill the old staging must finish first
  RA_HIP(hipDeviceSynchronize());
  if (c->stage && c->stage_owned) RA_HIP(hipFree(c->stage));
  c->stage = ptr;
  c->stage_cap = bytes;
  c->stage_owned = (ptr == nullptr);
  return RA_OK;
}

int mfma_rate(int iters, float* sink, double* tflops, hipStream_t stream) {
  if (iters < 1 || iters > (1 << 24)) return fail(RA_ERR_INVALID_ARG, "iters %d outside [1, 2^24]", iters);
  if (!sink || !tflops) return fail(RA_ERR_INVALID_ARG, "sink and tflops must be non-NULL");
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = launch_mfma_rate(iters / 8 + 1, sink, RA_MFMA_RATE_SINK_FLOATS, stream);  // warm-up
  if (e == hipSuccess) e = hipEventRecord(e0, stream);
  if (e == hipSuccess) e = launch_mfma_rate(iters, sink, RA_MFMA_RATE_SINK_FLOATS, stream);
  if (e == hipSuccess) e = hipEventRecord(e1, stream);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) return fail(RA_ERR_HIP, "mfma rate probe: %s", hipGetErrorString(e));
  // 8 waves per workgroup, 4 MFMAs of 32x32x16 (2*16384 flop) per wave and iteration
  const double flop = (double)RA_MFMA_RATE_SINK_FLOATS * 8.0 * 4.0 * 32768.0 * iters;
  *tflops = flop / (ms * 1e-3) / 1e12;
  return RA_OK;
}

void shutdown_all() {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ctx.empty()) (void)hipDeviceSynchronize();
  for (Ctx* c : g_ctx) {
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(c->device);
    (void)hipDeviceSynchronize();
    if (c->stage && c->stage_owned) (void)hipFree(c->stage);
    if (c->bwd) (void)hipFree(c->bwd);
    if (c->dec) (void)hipFree(c->dec);
    if (c->ffn) (void)hipFree(c->ffn);
    hipEvent_t evs[] = {c->ev_entry,   c->ev_side_end, c->ev_copied[0], c->ev_copied[1],
                        c->ev_done[0], c->ev_done[1],  c->ev_last};
    for (hipEvent_t e : evs)
      if (e) (void)hipEventDestroy(e);
    if (c->side) (void)hipStreamDestroy(c->side);
    (void)hipSetDevice(prev);
    delete c;
  }
  g_ctx.clear();
  for (auto& r : g_prof_recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof_recs.clear();
  for (hipEvent_t e : g_prof_pool) (void)hipEventDestroy(e);
  g_prof_pool.clear();
}

const char* last_error() { return g_last_error.c_str(); }
void clear_error() { g_last_error.clear(); }

}  // namespace ra

// ====================================================================== C ABI
extern "C" {

static ra::Shape make_shape(int n_blocks, int block_len, int heads, int kv_heads, int head_dim, int causal,
                            int rank, int elem_bytes) {
  ra::Shape s;
  s.n_blocks = n_blocks;
  s.block_len = block_len;
  s.heads = heads;
  s.kv_heads = kv_heads;
  s.head_dim = head_dim;
  s.causal = causal ? 1 : 0;
  s.rank = rank;
  s.elem_bytes = elem_bytes;
  return s;
}

int ring_attn_fwd(const void* q, const void* const* k_blocks, const void* const* v_blocks, int n_blocks,
                  int block_len, int heads, int kv_heads, int head_dim, int causal, int rank, float* out,
                  float* lse, ra_stream_t stream) {
  ra::clear_error();
  return ra::fwd_impl(q, k_blocks, v_blocks,
                      make_shape(n_blocks, block_len, heads, kv_heads, head_dim, causal, rank, 2), out, lse,
                      (hipStream_t)stream);
}

int ring_attn_fwd_f32(const float* q, const float* const* k_blocks, const float* const* v_blocks,
                      int n_blocks, int block_len, int heads, int kv_heads, int head_dim, int causal, int rank,
                      float* out, float* lse, ra_stream_t stream) {
  ra::clear_error();
  return ra::fwd_impl(q, (const void* const*)k_blocks, (const void* const*)v_blocks,
                      make_shape(n_blocks, block_len, heads, kv_heads, head_dim, causal, rank, 4), out, lse,
                      (hipStream_t)stream);
}

int ring_attn_merge(const float* out_a, const float* lse_a, const float* out_b, const float* lse_b, int rows,
                    int heads, int head_dim, float* out, float* lse, ra_stream_t stream) {
  ra::clear_error();
  return ra::merge_impl(out_a, lse_a, out_b, lse_b, rows, heads, head_dim, out, lse, (hipStream_t)stream);
}

int ring_attn_bwd(const void* q, const void* const* k_blocks, const void* const* v_blocks, const float* out,
                  const void* dout, const float* lse, int n_blocks, int block_len, int heads, int kv_heads,
                  int head_dim, int causal, int rank, float* dq, float* const* dk_blocks,
                  float* const* dv_blocks, ra_stream_t stream) {
  ra::clear_error();
  return ra::bwd_impl(q, k_blocks, v_blocks, out, dout, lse,
                      make_shape(n_blocks, block_len, heads, kv_heads, head_dim, causal, rank, 2), dq,
                      dk_blocks, dv_blocks, (hipStream_t)stream);
}

int ring_attn_bwd_f32(const float* q, const float* const* k_blocks, const float* const* v_blocks,
                      const float* out, const float* dout, const float* lse, int n_blocks, int block_len,
                      int heads, int kv_heads, int head_dim, int causal, int rank, float* dq,
                      float* const* dk_blocks, float* const* dv_blocks, ra_stream_t stream) {
  ra::clear_error();
  return ra::bwd_impl(q, (const void* const*)k_blocks, (const void* const*)v_blocks, out, dout, lse,
                      make_shape(n_blocks, block_len, heads, kv_heads, head_dim, causal, rank, 4), dq,
                      dk_blocks, dv_blocks, (hipStream_t)stream);
}

int ring_attn_fwd_zigzag(const void* q, const void* const* k_blocks, const void* const* v_blocks, int n_blocks,
                         int block_len, int heads, int kv_heads, int head_dim, int causal, int rank, float* out,
                         float* lse, ra_stream_t stream) {
  ra::clear_error();
  ra::Shape sh = make_shape(n_blocks, block_len, heads, kv_heads, head_dim, causal, rank, 2);
  sh.zigzag = 1;
  return ra::fwd_impl(q, k_blocks, v_blocks, sh, out, lse, (hipStream_t)stream);
}

int ring_attn_bwd_zigzag(const void* q, const void* const* k_blocks, const void* const* v_blocks, const float* out,
                         const void* dout, const float* lse, int n_blocks, int block_len, int heads, int kv_heads,
                         int head_dim, int causal, int rank, float* dq, float* const* dk_blocks,
                         float* const* dv_blocks, ra_stream_t stream) {
  ra::clear_error();
  ra::Shape sh = make_shape(n_blocks, block_len, heads, kv_heads, head_dim, causal, rank, 2);
  sh.zigzag = 1;
  return ra::bwd_impl(q, k_blocks, v_blocks, out, dout, lse, sh, dq, dk_blocks, dv_blocks, (hipStream_t)stream);
}

int ring_attn_schedule(int rank, int n_blocks, int causal, int* steps, int max_steps) {
  ra::clear_error();
  if (n_blocks < 1 || rank < 0 || rank >= n_blocks)
    return -ra::fail(RA_ERR_INVALID_ARG, "schedule: rank %d / n_blocks %d invalid", rank, n_blocks);
  const std::vector<int> s = ra::ring_schedule(rank, n_blocks, causal);
  if (steps) {
    if (max_steps < (int)s.size())
      return -ra::fail(RA_ERR_INVALID_ARG, "schedule: steps holds %d < %d entries", max_steps, (int)s.size());
    for (size_t i = 0; i < s.size(); ++i) steps[i] = s[i];
  }
  return (int)s.size();
}

int ring_attn_debug(int poison, long long delay_cycles) {
  ra::clear_error();
  return ra::debug_set(poison, delay_cycles);
}

const char* ring_attn_last_error(void) { return ra::last_error(); }

size_t ring_attn_workspace_bytes(int block_len, int kv_heads, int head_dim, int elem_bytes) {
  if (block_len < 1 || kv_heads < 1 || head_dim < 1 || (elem_bytes != 2 && elem_bytes != 4)) return 0;
  return 4 * (size_t)block_len * kv_heads * head_dim * elem_bytes;
}

int ring_attn_set_workspace(void* dev_ptr, size_t bytes) {
  ra::clear_error();
  return ra::set_workspace(dev_ptr, bytes);
}

int ring_attn_decode(const void* q, const void* const* k_blocks, const void* const* v_blocks, int n_blocks,
                     int block_len, int q_len, int heads, int kv_heads, int head_dim, long long q_pos0, float* out,
                     float* lse, ra_stream_t stream) {
  ra::clear_error();
  return ra::decode_impl(q, k_blocks, v_blocks, n_blocks, block_len, q_len, heads, kv_heads, head_dim, q_pos0, out,
                         lse, (hipStream_t)stream, false);
}

int ring_attn_decode_noalloc(const void* q, const void* const* k_blocks, const void* const* v_blocks, int n_blocks,
                             int block_len, int q_len, int heads, int kv_heads, int head_dim, long long q_pos0,
                             float* out, float* lse, ra_stream_t stream) {
  ra::clear_error();
  return ra::decode_impl(q, k_blocks, v_blocks, n_blocks, block_len, q_len, heads, kv_heads, head_dim, q_pos0, out,
                         lse, (hipStream_t)stream, true);
}

int ring_attn_ffn_blockwise(const void* x, const void* w1, const float* b1, const void* w2, const float* b2, int rows,
                            int hidden, int ffn, int chunk_rows, float* y, ra_stream_t stream) {
  ra::clear_error();
  return ra::ffn_impl(x, w1, b1, w2, b2, rows, hidden, ffn, chunk_rows, y, (hipStream_t)stream);
}

int ring_attn_mfma_rate(int iters, float* sink, double* tflops, ra_stream_t stream) {
  ra::clear_error();
  return ra::mfma_rate(iters, sink, tflops, (hipStream_t)stream);
}

int ring_attn_profile_enable(int enable) { return ra::profile_enable(enable); }

int ring_attn_profile_read(double* ms, int* count, double* copy_ms, double* hidden_ms) {
  ra::clear_error();
  return ra::profile_read(ms, count, copy_ms, hidden_ms);
}

void ring_attn_shutdown(void) { ra::shutdown_all(); }

}  // extern "C"
