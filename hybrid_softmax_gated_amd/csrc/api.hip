// C ABI of libarl2 (include/arl2.h): argument validation, workspace layout
// and the launch sequence of one ARL2 layer pass.
//
// Pass structure ("Technical Summary: Attend Locally, Remember Linearly
// (ARL2)", section 2.2): every pass computes out = O_intra + Q' S_{N-1};
// only the clean pass (update_flag = 1) then updates S. On the bf16 d = 128
// path a pass is two launches, in stream order:
//   1. intra-frame attention partials over key ranges       -> workspace
//      S16 := bf16(S), the copy the inter-frame read uses    -> workspace
//      (clean pass) per-chunk dS_c = K'^T diag(beta)(V' - K'S) -> workspace
//   2. merge partials + Q' = L2norm(q W_q), O_inter = Q' S16  -> out
//      (clean pass) S = alpha S + sum_c dS_c, in place
// Launch 1 only reads S; in launch 2 the read goes through S16, written in
// launch 1, so every token of the frame reads the pre-update state while S
// itself is updated.
#include "arl2.h"

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "arl2_kernels.h"

namespace arl2 {
thread_local LaunchTiming *g_launch_timing = nullptr;
}  // namespace arl2

namespace {

constexpr int32_t kMagic = 0x41524c32;  // "ARL2"
constexpr int64_t kMaxH = 65535;
constexpr int64_t kMaxB = 65535;

thread_local char g_err[512] = "";

arl2_status fail(arl2_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
arl2_status fail(arl2_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

arl2_status ok() {
  g_err[0] = 0;
  return ARL2_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Range {
  uintptr_t lo, hi;
};
Range range(const void *p, size_t bytes) { return {(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

size_t esize(int32_t dtype) { return dtype == ARL2_BF16 ? 2 : 4; }

bool mfma_path(int32_t d, int32_t dtype) { return d == ARL2_D_LARGE && dtype == ARL2_BF16; }

arl2_status check_shape(int64_t B, int64_t H, int64_t d, int64_t L, int64_t dtype,
                        const char *what) {
  if (dtype != ARL2_BF16 && dtype != ARL2_F32)
    return fail(ARL2_ERR_INVALID_ARG, "%s: dtype %lld is not ARL2_BF16 or ARL2_F32", what,
                (long long)dtype);
  if (B < 1 || B > kMaxB || H < 1 || H > kMaxH || L < 1 || L > ARL2_MAX_L || d < 1)
    return fail(ARL2_ERR_INVALID_ARG, "%s: bad shape B=%lld H=%lld d=%lld L=%lld", what,
                (long long)B, (long long)H, (long long)d, (long long)L);
  if (d != ARL2_D_SMALL && d != ARL2_D_LARGE)
    return fail(ARL2_ERR_UNSUPPORTED, "%s: head dimension %lld (supported: 16, 128)", what,
                (long long)d);
  if (B * L * H * d > ((int64_t)1 << 40))
    return fail(ARL2_ERR_INVALID_ARG, "%s: tensor of B*L*H*d = %lld elements is too large", what,
                (long long)(B * L * H * d));
  return ARL2_OK;
}

// Workspace layout of arl2_frame_forward.
struct FramePlan {
  bool mfma = false;
  arl2::AttnPlan ap;
  int chunk = 0, nchunk = 0;  // tokens per delta chunk, chunks per frame
  size_t off_o = 0, off_ml = 0, off_ds = 0, off_s16 = 0, total = 0;
};

FramePlan plan_frame(int64_t B, int64_t H, int64_t d, int64_t L, int32_t dtype) {
  FramePlan fp;
  fp.mfma = mfma_path((int32_t)d, dtype);
  size_t o_bytes, ml_bytes;
  if (fp.mfma) {
    fp.ap = arl2::plan_attention(B, H, L, L);
    const size_t blocks = (size_t)B * H * fp.ap.nqblk * fp.ap.nsplit;
    o_bytes = blocks * arl2::kPartialOBytes;
    ml_bytes = blocks * arl2::kPartialML * sizeof(float);
    fp.chunk = arl2::delta_chunk_tokens(B, H, L);
    fp.nchunk = (int)((L + fp.chunk - 1) / fp.chunk);
  } else {
    o_bytes = (size_t)B * H * L * d * sizeof(float);
    ml_bytes = 0;
    fp.chunk = arl2::kGenChunk;
    fp.nchunk = (int)((L + arl2::kGenChunk - 1) / arl2::kGenChunk);
  }
  const size_t ds_bytes = (size_t)B * H * fp.nchunk * d * d * sizeof(float);
  // The bf16 copy of the state that the inter-frame read uses (MFMA path).
  const size_t s16_bytes = fp.mfma ? (size_t)B * H * d * d * 2 : 0;
  fp.off_o = 0;
  fp.off_ml = align256(o_bytes);
  fp.off_ds = fp.off_ml + align256(ml_bytes);
  fp.off_s16 = fp.off_ds + align256(ds_bytes);
  fp.total = fp.off_s16 + align256(s16_bytes);
  return fp;
}

struct AttnOnlyPlan {
  bool mfma = false;
  arl2::AttnPlan ap;
  size_t off_o = 0, off_ml = 0, total = 0;
};

AttnOnlyPlan plan_attn_only(int64_t B, int64_t H, int64_t d, int64_t Lq, int64_t Lk,
                            int32_t dtype) {
  AttnOnlyPlan p;
  p.mfma = mfma_path((int32_t)d, dtype);
  size_t o_bytes, ml_bytes = 0;
  if (p.mfma) {
    p.ap = arl2::plan_attention(B, H, Lq, Lk);
    const size_t blocks = (size_t)B * H * p.ap.nqblk * p.ap.nsplit;
    o_bytes = blocks * arl2::kPartialOBytes;
    ml_bytes = blocks * arl2::kPartialML * sizeof(float);
  } else {
    o_bytes = (size_t)B * H * Lq * d * sizeof(float);
  }
  p.off_o = 0;
  p.off_ml = align256(o_bytes);
  p.total = p.off_ml + align256(ml_bytes);
  return p;
}

// ------------------------------------------------------------ kernel timing
struct Profiler {
  std::mutex mu;
  bool on = false;
  int repeat = 1;  // launches of an idempotent kernel between one event pair
  struct Rec {
    int count;
    size_t kernel;
    hipEvent_t a, b;
  };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> spare;
  std::vector<std::string> names;
  std::vector<int64_t> launches;
  std::vector<double> total_ms;

  hipError_t event(hipEvent_t *e) {
    if (!spare.empty()) {
      *e = spare.back();
      spare.pop_back();
      return hipSuccess;
    }
    return hipEventCreate(e);
  }
  size_t id(const char *name) {
    for (size_t i = 0; i < names.size(); ++i)
      if (names[i] == name) return i;
    names.emplace_back(name);
    launches.push_back(0);
    total_ms.push_back(0.0);
    return names.size() - 1;
  }
  // Wait for every recorded pair and fold it into the totals.
  hipError_t drain() {
    hipError_t err = hipSuccess;
    for (const Rec &r : pending) {
      float ms = 0.f;
      hipError_t e = hipEventSynchronize(r.b);
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
      if (e == hipSuccess) {
        launches[r.kernel] += r.count;
        total_ms[r.kernel] += ms;
      } else if (err == hipSuccess) {
        err = e;
      }
      spare.push_back(r.a);
      spare.push_back(r.b);
    }
    pending.clear();
    return err;
  }
};

Profiler &profiler() {
  static Profiler p;
  return p;
}

// Launch through `fn`, timed when profiling is on. With repeat = 1, or for
// a kernel that updates memory it reads (not idempotent), the two events are
// taken from the kernels' own start and end (arl2::launch with a timing
// region open), so the time is that of the launch in its place in the
// sequence. With repeat > 1 an idempotent launch is repeated back to back
// between two event markers, which spreads the markers' own overhead over
// the repeats (warm caches, no gaps to the neighbouring launches).
template <class F>
hipError_t timed(const char *name, hipStream_t s, F fn, bool idempotent = true) {
  Profiler &p = profiler();
  std::unique_lock<std::mutex> lk(p.mu);
  if (!p.on) {
    lk.unlock();
    return fn();
  }
  hipEvent_t a, b;
  hipError_t e = p.event(&a);
  if (e != hipSuccess) return e;
  if ((e = p.event(&b)) != hipSuccess) return e;
  const int count = idempotent ? p.repeat : 1;
  if (count == 1) {
    arl2::LaunchTiming lt{a, b, false};
    arl2::g_launch_timing = &lt;
    e = fn();
    arl2::g_launch_timing = nullptr;
    if (e != hipSuccess) return e;
    if (!lt.started) return hipErrorInvalidValue;  // nothing was launched
  } else {
    if ((e = hipEventRecord(a, s)) != hipSuccess) return e;
    for (int i = 0; i < count; ++i)
      if ((e = fn()) != hipSuccess) return e;
    if ((e = hipEventRecord(b, s)) != hipSuccess) return e;
  }
  p.pending.push_back({count, p.id(name), a, b});
  return hipSuccess;
}

arl2_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ARL2_OK;
  return fail(ARL2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

// Scratch of arl2_frame_forward_noalloc: the pass's workspace (attention
// partials and update partials), one copy per device, held until the
// process ends. Host code never uses this name as an address: each
// device's copy is reached through the address hipGetSymbolAddress gives
// with that device current (scratch_address below).
static __device__ __align__(256) char scratch[ARL2_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The current device's address of `scratch`, looked up once per device.
arl2_status scratch_address(const char *fn, void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ARL2_ERR_UNSUPPORTED, "%s: device index %d (at most %d devices)", fn, dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, fn);
    if (!p || !aligned(p, 256))
      return fail(ARL2_ERR_HIP, "%s: the scratch of device %d has no 256-byte aligned address",
                  fn, dev);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ARL2_OK;
}

}  // namespace

extern "C" {

int32_t arl2_version(void) { return ARL2_VERSION; }

const char *arl2_status_string(int32_t status) {
  switch (status) {
    case ARL2_OK: return "ok";
    case ARL2_ERR_INVALID_ARG: return "invalid argument";
    case ARL2_ERR_UNSUPPORTED: return "unsupported";
    case ARL2_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *arl2_last_error(void) { return g_err; }

size_t arl2_workspace_bytes(int32_t B, int32_t H, int32_t d, int32_t L, int32_t dtype) {
  if (check_shape(B, H, d, L, dtype, "arl2_workspace_bytes") != ARL2_OK) return 0;
  return plan_frame(B, H, d, L, dtype).total;
}

arl2_status arl2_state_init(arl2_state *st, int32_t B, int32_t H, int32_t d, int32_t L,
                            int32_t dtype, float *S_dev, void *ws_dev, size_t ws_bytes,
                            void *stream) {
  if (!st) return fail(ARL2_ERR_INVALID_ARG, "arl2_state_init: st is NULL");
  arl2_status cs = check_shape(B, H, d, L, dtype, "arl2_state_init");
  if (cs != ARL2_OK) return cs;
  if (!S_dev) return fail(ARL2_ERR_INVALID_ARG, "arl2_state_init: S_dev is NULL");
  if (!aligned(S_dev, 16))
    return fail(ARL2_ERR_INVALID_ARG, "arl2_state_init: S_dev is not 16-byte aligned");
  const size_t need = plan_frame(B, H, d, L, dtype).total;
  // No workspace at all (NULL, 0 bytes): the state can only run passes
  // through arl2_frame_forward_noalloc, whose scratch is the library's own.
  const bool no_ws = !ws_dev && ws_bytes == 0;
  if (!no_ws && ws_bytes < need)
    return fail(ARL2_ERR_INVALID_ARG, "arl2_state_init: workspace of %zu bytes, need %zu",
                ws_bytes, need);
  if (!no_ws && need > 0 && !ws_dev)
    return fail(ARL2_ERR_INVALID_ARG, "arl2_state_init: ws_dev is NULL");
  if (ws_dev && !aligned(ws_dev, 256))
    return fail(ARL2_ERR_INVALID_ARG, "arl2_state_init: ws_dev is not 256-byte aligned");
  const size_t s_bytes = (size_t)B * H * d * d * sizeof(float);
  if (ws_dev && overlap(range(S_dev, s_bytes), range(ws_dev, ws_bytes)))
    return fail(ARL2_ERR_INVALID_ARG, "arl2_state_init: S and workspace overlap");
  if (no_ws) {
    // Set-up of a caller that cannot allocate: find this device's scratch
    // now, so that its passes do not have to.
    void *p = nullptr;
    arl2_status ss = scratch_address("arl2_state_init", &p);
    if (ss != ARL2_OK) return ss;
  }
  arl2_status hs = hip_status(
      timed("fill_state", (hipStream_t)stream, [&] { return arl2::launch_fill_state(S_dev, nullptr, (int64_t)B * H * d * d, (hipStream_t)stream); }),
      "arl2_state_init");
  if (hs != ARL2_OK) return hs;
  st->B = B;
  st->H = H;
  st->d = d;
  st->L = L;
  st->dtype = dtype;
  st->magic = kMagic;
  st->S = S_dev;
  st->ws = ws_dev;
  st->ws_bytes = ws_bytes;
  return ok();
}

static arl2_status check_state(const arl2_state *st, const char *what) {
  if (!st) return fail(ARL2_ERR_INVALID_ARG, "%s: st is NULL", what);
  if (st->magic != kMagic || !st->S)
    return fail(ARL2_ERR_INVALID_ARG, "%s: state was not set up by arl2_state_init", what);
  return check_shape(st->B, st->H, st->d, st->L, st->dtype, what);
}

// The state's own workspace must hold the frame plan (passes other than
// arl2_frame_forward_noalloc use it).
static arl2_status check_state_ws(const arl2_state *st, const char *what) {
  if (st->ws_bytes < plan_frame(st->B, st->H, st->d, st->L, st->dtype).total)
    return fail(ARL2_ERR_INVALID_ARG,
                "%s: the state's workspace is too small for its shape (a state bound without "
                "a workspace runs passes through arl2_frame_forward_noalloc only)", what);
  return ARL2_OK;
}

arl2_status arl2_state_reset(arl2_state *st, const float *S0_dev, void *stream) {
  arl2_status cs = check_state(st, "arl2_state_reset");
  if (cs != ARL2_OK) return cs;
  const int64_t n = (int64_t)st->B * st->H * st->d * st->d;
  if (S0_dev) {
    if (!aligned(S0_dev, 4))
      return fail(ARL2_ERR_INVALID_ARG, "arl2_state_reset: S0 is misaligned");
    if (overlap(range(S0_dev, n * sizeof(float)), range(st->S, n * sizeof(float))))
      return fail(ARL2_ERR_INVALID_ARG, "arl2_state_reset: S0 overlaps S");
  }
  arl2_status hs = hip_status(timed("fill_state", (hipStream_t)stream, [&] { return arl2::launch_fill_state(st->S, S0_dev, n, (hipStream_t)stream); }),
                              "arl2_state_reset");
  if (hs != ARL2_OK) return hs;
  return ok();
}

namespace {

// Argument checks of one pass whose workspace is `ws_base`, `ws_cap` bytes
// (the state's own, or the no-allocation scratch; an empty range when that
// is not known yet). No HIP call.
arl2_status check_frame_args(const char *fn, const void *q, const void *k, const void *v,
                             const void *Wphi, const arl2_state *st, const float *alpha,
                             int32_t gate, const float *beta, const void *out,
                             int32_t update_flag, const void *ws_base, size_t ws_cap) {
  if (update_flag != 0 && update_flag != 1)
    return fail(ARL2_ERR_INVALID_ARG, "%s: update_flag %d is not 0 or 1", fn, update_flag);
  if (gate != ARL2_GATE_HEADWISE && gate != ARL2_GATE_ELEMENTWISE)
    return fail(ARL2_ERR_INVALID_ARG, "%s: gate %d is not a gate kind", fn, gate);
  const void *tens[5] = {q, k, v, Wphi, out};
  const char *names[5] = {"q", "k", "v", "Wphi", "out"};
  for (int i = 0; i < 5; ++i) {
    if (!tens[i]) return fail(ARL2_ERR_INVALID_ARG, "%s: %s is NULL", fn, names[i]);
    if (!aligned(tens[i], 16))
      return fail(ARL2_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, names[i]);
  }
  const int64_t B = st->B, H = st->H, d = st->d, L = st->L;
  const size_t es = esize(st->dtype);
  const size_t act = (size_t)B * L * H * d * es;
  const size_t wbytes = (size_t)3 * H * d * d * es;
  const size_t sbytes = (size_t)B * H * d * d * sizeof(float);
  const Range r_out = range(out, act), r_S = range(st->S, sbytes), r_ws = range(ws_base, ws_cap);
  const Range r_in[4] = {range(q, act), range(k, act), range(v, act), range(Wphi, wbytes)};
  for (int i = 0; i < 4; ++i)
    if (overlap(r_out, r_in[i]))
      return fail(ARL2_ERR_INVALID_ARG, "%s: out overlaps %s", fn, names[i]);
  if (overlap(r_out, r_S) || overlap(r_out, r_ws))
    return fail(ARL2_ERR_INVALID_ARG, "%s: out overlaps the state or its workspace", fn);
  for (int i = 0; i < 4; ++i)
    if (overlap(r_ws, r_in[i]) || overlap(r_S, r_in[i]))
      return fail(ARL2_ERR_INVALID_ARG, "%s: %s overlaps the state or its workspace", fn,
                  names[i]);
  if (update_flag) {
    if (!alpha || !beta)
      return fail(ARL2_ERR_INVALID_ARG, "%s: alpha and beta are required when update_flag == 1",
                  fn);
    if (!aligned(alpha, 4) || !aligned(beta, 4))
      return fail(ARL2_ERR_INVALID_ARG, "%s: alpha/beta are misaligned", fn);
    const size_t abytes = (size_t)B * H * (gate == ARL2_GATE_ELEMENTWISE ? d : 1) * 4;
    const Range r_a = range(alpha, abytes), r_b = range(beta, (size_t)B * L * H * 4);
    if (overlap(r_a, r_S) || overlap(r_b, r_S) || overlap(r_a, r_ws) || overlap(r_b, r_ws))
      return fail(ARL2_ERR_INVALID_ARG, "%s: alpha/beta overlap the state or its workspace", fn);
    // The output is written in the launch whose update items read beta, and
    // before the launch that reads alpha: an overlap would corrupt S.
    if (overlap(r_out, r_a) || overlap(r_out, r_b))
      return fail(ARL2_ERR_INVALID_ARG, "%s: out overlaps alpha/beta", fn);
  }
  return ARL2_OK;
}

// One pass with the workspace `ws_base` of `ws_cap` bytes (the state's own,
// or the no-allocation scratch).
arl2_status frame_forward_impl(const char *fn, const void *q, const void *k, const void *v,
                               const void *Wphi, arl2_state *st, const float *alpha,
                               int32_t gate, const float *beta, void *out, int32_t update_flag,
                               void *ws_base, size_t ws_cap, void *stream) {
  arl2_status cs = check_frame_args(fn, q, k, v, Wphi, st, alpha, gate, beta, out, update_flag,
                                    ws_base, ws_cap);
  if (cs != ARL2_OK) return cs;
  const int64_t B = st->B, H = st->H, d = st->d, L = st->L;
  const size_t es = esize(st->dtype);
  hipStream_t s = (hipStream_t)stream;
  const FramePlan fp = plan_frame(B, H, d, L, st->dtype);
  char *ws = (char *)ws_base;
  float *ws_o = (float *)(ws + fp.off_o);
  float *ws_ml = (float *)(ws + fp.off_ml);
  float *ws_ds = (float *)(ws + fp.off_ds);
  void *ws_s16 = ws + fp.off_s16;
  const char *wbase = (const char *)Wphi;
  const void *Wq = wbase;
  const void *Wk = wbase + (size_t)H * d * d * es;
  const void *Wv = wbase + (size_t)2 * H * d * d * es;

  const int iB = (int)B, iH = (int)H, iL = (int)L, id = (int)d, dt = st->dtype;
  float *S = st->S;
  hipError_t e;
  if (fp.mfma) {
    const arl2::AttnArgs aa{q, k, v, iB, iH, iL, iL, fp.ap, ws_o, ws_ml};
    const arl2::CombineArgs ca{ws_o, ws_ml, q, Wq, ws_s16, iB, iH, iL, fp.ap, out};
    const arl2::DeltaArgs da{k, v, Wk, Wv, S, beta, iB, iH, iL, fp.chunk, fp.nchunk, ws_ds};
    const arl2::ApplyArgs ap{S, alpha, gate == ARL2_GATE_ELEMENTWISE, ws_ds, iB, iH, fp.nchunk};
    const int64_t nstate = B * H * d * d;
    if ((e = timed(update_flag ? "attn_delta" : "attn_partial", s, [&] {
           return arl2::launch_pass_head_bf16(aa, update_flag ? &da : nullptr, S, ws_s16, nstate,
                                              s);
         })))
      return hip_status(e, fn);
    if ((e = timed(update_flag ? "combine_apply" : "combine", s, [&] {
           return arl2::launch_tail_bf16(ca, update_flag ? &ap : nullptr, s);
         }, /*idempotent=*/update_flag == 0)))
      return hip_status(e, fn);
    return ok();
  } else {
    if ((e = timed("generic_attention", s, [&] {
           return arl2::launch_generic_attention(dt, id, q, k, v, iB, iH, iL, iL, ws_o, s);
         })))
      return hip_status(e, fn);
    if ((e = timed("generic_inter_combine", s, [&] {
           return arl2::launch_generic_inter_combine(dt, id, q, Wq, S, ws_o, iB, iH, iL, out, true,
                                                     s);
         })))
      return hip_status(e, fn);
    if (update_flag) {
      if ((e = timed("generic_delta_partial", s, [&] {
             return arl2::launch_generic_delta_partial(dt, id, k, v, Wk, Wv, S, beta, iB, iH, iL,
                                                       ws_ds, s);
           })))
        return hip_status(e, fn);
    }
  }
  if (update_flag) {
    if ((e = timed("delta_apply", s, [&] {
           return arl2::launch_delta_apply(S, alpha, gate == ARL2_GATE_ELEMENTWISE, ws_ds, iB, iH,
                                           id, fp.nchunk, s);
         }, /*idempotent=*/false)))
      return hip_status(e, fn);
  }
  return ok();
}

}  // namespace

arl2_status arl2_frame_forward(const void *q, const void *k, const void *v, const void *Wphi,
                               arl2_state *st, const float *alpha, const float *beta, void *out,
                               int32_t update_flag, void *stream) {
  const char *fn = "arl2_frame_forward";
  arl2_status cs = check_state(st, fn);
  if (cs == ARL2_OK) cs = check_state_ws(st, fn);
  if (cs != ARL2_OK) return cs;
  return frame_forward_impl(fn, q, k, v, Wphi, st, alpha, ARL2_GATE_HEADWISE, beta, out,
                            update_flag, st->ws, st->ws_bytes, stream);
}

arl2_status arl2_frame_forward_gated(const void *q, const void *k, const void *v,
                                     const void *Wphi, arl2_state *st, const float *alpha,
                                     int32_t gate, const float *beta, void *out,
                                     int32_t update_flag, void *stream) {
  const char *fn = "arl2_frame_forward_gated";
  arl2_status cs = check_state(st, fn);
  if (cs == ARL2_OK) cs = check_state_ws(st, fn);
  if (cs != ARL2_OK) return cs;
  return frame_forward_impl(fn, q, k, v, Wphi, st, alpha, gate, beta, out, update_flag, st->ws,
                            st->ws_bytes, stream);
}

arl2_status arl2_frame_forward_noalloc(const void *q, const void *k, const void *v,
                                       const void *Wphi, arl2_state *st, const float *alpha,
                                       const float *beta, void *out, int32_t update_flag,
                                       void *stream) {
  const char *fn = "arl2_frame_forward_noalloc";
  arl2_status cs = check_state(st, fn);
  if (cs != ARL2_OK) return cs;
  const size_t need = plan_frame(st->B, st->H, st->d, st->L, st->dtype).total;
  if (need > ARL2_NOALLOC_SCRATCH_BYTES)
    return fail(ARL2_ERR_INVALID_ARG,
                "%s: this shape needs %zu bytes of scratch; the no-allocation pass holds at most "
                "%zu (B=%d H=%d d=%d L=%d): use arl2_frame_forward with a workspace",
                fn, need, (size_t)ARL2_NOALLOC_SCRATCH_BYTES, st->B, st->H, st->d, st->L);
  cs = check_frame_args(fn, q, k, v, Wphi, st, alpha, ARL2_GATE_HEADWISE, beta, out,
                        update_flag, nullptr, 0);
  if (cs != ARL2_OK) return cs;
  void *scr = nullptr;
  cs = scratch_address(fn, &scr);
  if (cs != ARL2_OK) return cs;
  return frame_forward_impl(fn, q, k, v, Wphi, st, alpha, ARL2_GATE_HEADWISE, beta, out,
                            update_flag, scr, ARL2_NOALLOC_SCRATCH_BYTES, stream);
}

namespace {

// Token-level workspace: chunk records, then O_inter (MFMA path only).
struct TokenPlan {
  size_t off_oi = 0, total = 0;
};
TokenPlan plan_token(int64_t B, int64_t H, int64_t d, int64_t L, int32_t dtype) {
  TokenPlan tp;
  if (!mfma_path((int32_t)d, dtype)) return tp;
  const int64_t nchunk = (L + arl2::kTokenChunk - 1) / arl2::kTokenChunk;
  tp.off_oi = align256((size_t)B * H * nchunk * arl2::kTokenRecordBytes);
  tp.total = tp.off_oi + align256((size_t)B * L * H * d * sizeof(float));
  return tp;
}

}  // namespace

size_t arl2_token_level_workspace_bytes(int32_t B, int32_t H, int32_t d, int32_t L,
                                        int32_t dtype) {
  if (check_shape(B, H, d, L, dtype, "arl2_token_level_workspace_bytes") != ARL2_OK) return 0;
  return plan_token(B, H, d, L, dtype).total;
}

arl2_status arl2_frame_forward_token_level(const void *q, const void *k, const void *v,
                                           const void *Wphi, arl2_state *st, const float *alpha,
                                           const float *beta, void *out, int32_t update_flag,
                                           void *tl_ws, size_t tl_ws_bytes, void *stream) {
  const char *fn = "arl2_frame_forward_token_level";
  arl2_status cs = check_state(st, fn);
  if (cs == ARL2_OK) cs = check_state_ws(st, fn);
  if (cs != ARL2_OK) return cs;
  if (update_flag != 0 && update_flag != 1)
    return fail(ARL2_ERR_INVALID_ARG, "%s: update_flag %d is not 0 or 1", fn, update_flag);
  const void *tens[5] = {q, k, v, Wphi, out};
  const char *names[5] = {"q", "k", "v", "Wphi", "out"};
  for (int i = 0; i < 5; ++i) {
    if (!tens[i]) return fail(ARL2_ERR_INVALID_ARG, "%s: %s is NULL", fn, names[i]);
    if (!aligned(tens[i], 16))
      return fail(ARL2_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, names[i]);
  }
  if (!alpha || !beta || !aligned(alpha, 4) || !aligned(beta, 4))
    return fail(ARL2_ERR_INVALID_ARG, "%s: alpha and beta are required on every pass", fn);
  const int64_t B = st->B, H = st->H, d = st->d, L = st->L;
  const TokenPlan tp = plan_token(B, H, d, L, st->dtype);
  if (tl_ws_bytes < tp.total)
    return fail(ARL2_ERR_INVALID_ARG, "%s: token-level workspace of %zu bytes, need %zu", fn,
                tl_ws_bytes, tp.total);
  if (tp.total > 0 && (!tl_ws || !aligned(tl_ws, 256)))
    return fail(ARL2_ERR_INVALID_ARG, "%s: tl_ws is NULL or not 256-byte aligned", fn);
  const size_t es = esize(st->dtype);
  const size_t act = (size_t)B * L * H * d * es;
  const Range r_out = range(out, act), r_S = range(st->S, (size_t)B * H * d * d * 4),
              r_ws = range(st->ws, st->ws_bytes),
              r_tl = tp.total ? range(tl_ws, tl_ws_bytes) : Range{0, 0};
  const Range r_in[6] = {range(q, act), range(k, act), range(v, act),
                         range(Wphi, (size_t)3 * H * d * d * es), range(alpha, (size_t)B * H * 4),
                         range(beta, (size_t)B * L * H * 4)};
  const char *in_names[6] = {"q", "k", "v", "Wphi", "alpha", "beta"};
  const Range r_w[4] = {r_out, r_S, r_ws, r_tl};
  const char *w_names[4] = {"out", "the state", "the state's workspace", "tl_ws"};
  for (int a = 0; a < 4; ++a) {
    for (int i = 0; i < 6; ++i)
      if (overlap(r_w[a], r_in[i]))
        return fail(ARL2_ERR_INVALID_ARG, "%s: %s overlaps %s", fn, w_names[a], in_names[i]);
    for (int c = 0; c < a; ++c)
      if (overlap(r_w[a], r_w[c]))
        return fail(ARL2_ERR_INVALID_ARG, "%s: %s overlaps %s", fn, w_names[a], w_names[c]);
  }

  hipStream_t s = (hipStream_t)stream;
  const FramePlan fp = plan_frame(B, H, d, L, st->dtype);
  char *ws = (char *)st->ws;
  float *ws_o = (float *)(ws + fp.off_o);
  float *ws_ml = (float *)(ws + fp.off_ml);
  const char *wbase = (const char *)Wphi;
  const void *Wq = wbase;
  const void *Wk = wbase + (size_t)H * d * d * es;
  const void *Wv = wbase + (size_t)2 * H * d * d * es;
  const int iB = (int)B, iH = (int)H, iL = (int)L, id = (int)d, dt = st->dtype;
  float *S = st->S;
  hipError_t e;
  if (fp.mfma) {
    float *o_inter = (float *)((char *)tl_ws + tp.off_oi);
    const arl2::AttnArgs aa{q, k, v, iB, iH, iL, iL, fp.ap, ws_o, ws_ml};
    const arl2::TokenLevelArgs ta{q, k, v, Wq, Wk, Wv, alpha, beta, S, iB, iH, iL, update_flag,
                                  tl_ws, o_inter};
    arl2::CombineArgs ca{ws_o, ws_ml, q, nullptr, nullptr, iB, iH, iL, fp.ap, out};
    ca.o_inter = o_inter;
    if ((e = timed("attn_partial", s, [&] { return arl2::launch_attn_partial_bf16(aa, s); })))
      return hip_status(e, fn);
    if ((e = timed("token_level", s, [&] { return arl2::launch_token_level_bf16(ta, s); },
                   /*idempotent=*/update_flag == 0)))
      return hip_status(e, fn);
    if ((e = timed("combine_token_level", s, [&] { return arl2::launch_tail_bf16(ca, nullptr, s); })))
      return hip_status(e, fn);
  } else {
    if ((e = timed("generic_attention", s, [&] {
           return arl2::launch_generic_attention(dt, id, q, k, v, iB, iH, iL, iL, ws_o, s);
         })))
      return hip_status(e, fn);
    if ((e = timed("generic_token_level", s, [&] {
           return arl2::launch_token_level_generic(dt, id, q, k, v, Wphi, ws_o, S, alpha, beta,
                                                   iB, iH, iL, update_flag, out, s);
         }, /*idempotent=*/update_flag == 0)))
      return hip_status(e, fn);
  }
  return ok();
}

size_t arl2_softmax_attention_workspace_bytes(int32_t B, int32_t H, int32_t d, int32_t Lq,
                                              int32_t Lk, int32_t dtype) {
  if (check_shape(B, H, d, Lq, dtype, "arl2_softmax_attention_workspace_bytes") != ARL2_OK ||
      check_shape(B, H, d, Lk, dtype, "arl2_softmax_attention_workspace_bytes") != ARL2_OK)
    return 0;
  return plan_attn_only(B, H, d, Lq, Lk, dtype).total;
}

arl2_status arl2_softmax_attention(const void *q, const void *kc, const void *vc, int32_t B,
                                   int32_t H, int32_t d, int32_t Lq, int32_t Lk, int32_t dtype,
                                   void *out, void *ws, size_t ws_bytes, void *stream) {
  const char *fn = "arl2_softmax_attention";
  arl2_status cs = check_shape(B, H, d, Lq, dtype, fn);
  if (cs != ARL2_OK) return cs;
  cs = check_shape(B, H, d, Lk, dtype, fn);
  if (cs != ARL2_OK) return cs;
  const void *tens[4] = {q, kc, vc, out};
  const char *names[4] = {"q", "kc", "vc", "out"};
  for (int i = 0; i < 4; ++i) {
    if (!tens[i]) return fail(ARL2_ERR_INVALID_ARG, "%s: %s is NULL", fn, names[i]);
    if (!aligned(tens[i], 16))
      return fail(ARL2_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, names[i]);
  }
  const AttnOnlyPlan ap = plan_attn_only(B, H, d, Lq, Lk, dtype);
  if (ws_bytes < ap.total)
    return fail(ARL2_ERR_INVALID_ARG, "%s: workspace of %zu bytes, need %zu", fn, ws_bytes,
                ap.total);
  if (!ws || !aligned(ws, 256))
    return fail(ARL2_ERR_INVALID_ARG, "%s: ws is NULL or not 256-byte aligned", fn);
  const size_t es = esize(dtype);
  const Range r_out = range(out, (size_t)B * Lq * H * d * es);
  const Range r_in[3] = {range(q, (size_t)B * Lq * H * d * es),
                         range(kc, (size_t)B * Lk * H * d * es),
                         range(vc, (size_t)B * Lk * H * d * es)};
  const Range r_ws = range(ws, ws_bytes);
  for (int i = 0; i < 3; ++i)
    if (overlap(r_out, r_in[i]) || overlap(r_ws, r_in[i]))
      return fail(ARL2_ERR_INVALID_ARG, "%s: %s overlaps out or the workspace", fn, names[i]);
  if (overlap(r_out, r_ws)) return fail(ARL2_ERR_INVALID_ARG, "%s: out overlaps ws", fn);

  hipStream_t s = (hipStream_t)stream;
  float *ws_o = (float *)((char *)ws + ap.off_o);
  float *ws_ml = (float *)((char *)ws + ap.off_ml);
  hipError_t e;
  if (ap.mfma) {
    const arl2::AttnArgs aa{q, kc, vc, B, H, Lq, Lk, ap.ap, ws_o, ws_ml};
    const arl2::CombineArgs ca{ws_o, ws_ml, q, nullptr, nullptr, B, H, Lq, ap.ap, out};
    if ((e = timed("attn_partial", s, [&] { return arl2::launch_attn_partial_bf16(aa, s); })))
      return hip_status(e, fn);
    if ((e = timed("combine", s, [&] { return arl2::launch_tail_bf16(ca, nullptr, s); })))
      return hip_status(e, fn);
  } else {
    if ((e = timed("generic_attention", s, [&] {
           return arl2::launch_generic_attention(dtype, d, q, kc, vc, B, H, Lq, Lk, ws_o, s);
         })))
      return hip_status(e, fn);
    if ((e = timed("generic_attn_merge", s, [&] {
           return arl2::launch_generic_inter_combine(dtype, d, q, nullptr, nullptr, ws_o, B, H, Lq,
                                                     out, false, s);
         })))
      return hip_status(e, fn);
  }
  return ok();
}

static arl2_status check_gate_shape(int64_t B, int64_t L, int64_t D, int64_t H, int64_t dtype,
                                    const char *what) {
  if (dtype != ARL2_BF16 && dtype != ARL2_F32)
    return fail(ARL2_ERR_INVALID_ARG, "%s: dtype %lld is not ARL2_BF16 or ARL2_F32", what,
                (long long)dtype);
  if (B < 1 || B > kMaxB || L < 1 || L > ARL2_MAX_L || D < 1 || D > ARL2_MAX_GATE_D || H < 1 ||
      H > kMaxH)
    return fail(ARL2_ERR_INVALID_ARG, "%s: bad shape B=%lld L=%lld D=%lld H=%lld", what,
                (long long)B, (long long)L, (long long)D, (long long)H);
  if (B * L * D > ((int64_t)1 << 40) || B * L * H > ((int64_t)1 << 36))
    return fail(ARL2_ERR_INVALID_ARG, "%s: B=%lld L=%lld D=%lld H=%lld is too large", what,
                (long long)B, (long long)L, (long long)D, (long long)H);
  return ARL2_OK;
}

size_t arl2_gate_projections_workspace_bytes(int32_t B, int32_t L, int32_t D, int32_t H,
                                             int32_t dtype) {
  if (check_gate_shape(B, L, D, H, dtype, "arl2_gate_projections_workspace_bytes") != ARL2_OK)
    return 0;
  return arl2::plan_gate(B, L, D, H, dtype).ws_bytes;
}

arl2_status arl2_gate_projections(const void *x, const void *Wa, const void *Wb, int32_t B,
                                  int32_t L, int32_t D, int32_t H, int32_t dtype, float *alpha,
                                  float *beta, void *ws, size_t ws_bytes, void *stream) {
  const char *fn = "arl2_gate_projections";
  arl2_status cs = check_gate_shape(B, L, D, H, dtype, fn);
  if (cs != ARL2_OK) return cs;
  const void *tens[3] = {x, Wa, Wb};
  const char *names[3] = {"x", "Wa", "Wb"};
  for (int i = 0; i < 3; ++i) {
    if (!tens[i]) return fail(ARL2_ERR_INVALID_ARG, "%s: %s is NULL", fn, names[i]);
    if (!aligned(tens[i], 16))
      return fail(ARL2_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, names[i]);
  }
  if (!alpha || !beta || !aligned(alpha, 4) || !aligned(beta, 4))
    return fail(ARL2_ERR_INVALID_ARG, "%s: alpha/beta are NULL or misaligned", fn);
  const arl2::GatePlan gp = arl2::plan_gate(B, L, D, H, dtype);
  const size_t need = gp.ws_bytes;
  if (ws_bytes < need)
    return fail(ARL2_ERR_INVALID_ARG, "%s: workspace of %zu bytes, need %zu", fn, ws_bytes, need);
  if (!ws || !aligned(ws, 256))
    return fail(ARL2_ERR_INVALID_ARG, "%s: ws is NULL or not 256-byte aligned", fn);
  const size_t es = esize(dtype);
  const Range r_in[3] = {range(x, (size_t)B * L * D * es), range(Wa, (size_t)H * D * es),
                         range(Wb, (size_t)H * D * es)};
  const Range r_out[3] = {range(alpha, (size_t)B * H * 4), range(beta, (size_t)B * L * H * 4),
                          range(ws, ws_bytes)};
  const char *onames[3] = {"alpha", "beta", "ws"};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 3; ++i)
      if (overlap(r_out[o], r_in[i]))
        return fail(ARL2_ERR_INVALID_ARG, "%s: %s overlaps %s", fn, onames[o], names[i]);
    for (int j = 0; j < o; ++j)
      if (overlap(r_out[o], r_out[j]))
        return fail(ARL2_ERR_INVALID_ARG, "%s: %s overlaps %s", fn, onames[o], onames[j]);
  }
  hipStream_t s = (hipStream_t)stream;
  const arl2::GateArgs ga{x, Wa, Wb, B, L, D, H, dtype, gp, ws, alpha, beta};
  hipError_t e;
  if ((e = timed("gate_projections", s, [&] { return arl2::launch_gate_projections(ga, s); })))
    return hip_status(e, fn);
  return ok();
}

arl2_status arl2_profile_enable(int32_t on, int32_t repeat) {
  if (repeat < 1 || repeat > 1000)
    return fail(ARL2_ERR_INVALID_ARG, "arl2_profile_enable: repeat %d not in [1, 1000]", repeat);
  Profiler &p = profiler();
  std::lock_guard<std::mutex> lk(p.mu);
  p.on = on != 0;
  p.repeat = repeat;
  return ok();
}

void arl2_profile_reset(void) {
  Profiler &p = profiler();
  std::lock_guard<std::mutex> lk(p.mu);
  // The pending timings are discarded anyway; an event error here has nothing to report to.
  (void)p.drain();
  for (size_t i = 0; i < p.names.size(); ++i) {
    p.launches[i] = 0;
    p.total_ms[i] = 0.0;
  }
}

arl2_status arl2_profile_report(char *buf, size_t len) {
  if (!buf || len == 0) return fail(ARL2_ERR_INVALID_ARG, "arl2_profile_report: no buffer");
  Profiler &p = profiler();
  std::lock_guard<std::mutex> lk(p.mu);
  const hipError_t e = p.drain();
  std::string txt;
  char line[160];
  for (size_t i = 0; i < p.names.size(); ++i) {
    snprintf(line, sizeof(line), "%s %lld %.6f\n", p.names[i].c_str(), (long long)p.launches[i],
             p.total_ms[i]);
    txt += line;
  }
  snprintf(buf, len, "%s", txt.c_str());
  if (e != hipSuccess) return hip_status(e, "arl2_profile_report");
  return ok();
}

arl2_status arl2_profile_mfma_peak(int32_t iters, double *tflops, void *stream) {
  static const char *fn = "arl2_profile_mfma_peak";
  if (!tflops) return fail(ARL2_ERR_INVALID_ARG, "%s: tflops is NULL", fn);
  if (iters < 1 || iters > (1 << 20))
    return fail(ARL2_ERR_INVALID_ARG, "%s: iters %d not in [1, 2^20]", fn, iters);
  hipStream_t s = (hipStream_t)stream;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (cus < 1) return fail(ARL2_ERR_HIP, "%s: no compute units reported", fn);
  float *sink = nullptr;
  hipEvent_t t0 = nullptr, t1 = nullptr;
  if ((e = hipMalloc((void **)&sink, (size_t)cus * 512 * sizeof(float))) != hipSuccess)
    return hip_status(e, fn);
  float ms = 0.f;
  if ((e = hipEventCreate(&t0)) == hipSuccess && (e = hipEventCreate(&t1)) == hipSuccess &&
      (e = arl2::launch_mfma_peak(cus, 16, sink, s)) == hipSuccess &&  // warm-up
      (e = hipEventRecord(t0, s)) == hipSuccess &&
      (e = arl2::launch_mfma_peak(cus, iters, sink, s)) == hipSuccess &&
      (e = hipEventRecord(t1, s)) == hipSuccess && (e = hipEventSynchronize(t1)) == hipSuccess)
    e = hipEventElapsedTime(&ms, t0, t1);
  if (t0) (void)hipEventDestroy(t0);
  if (t1) (void)hipEventDestroy(t1);
  (void)hipFree(sink);
  if (e != hipSuccess) return hip_status(e, fn);
  if (!(ms > 0.f)) return fail(ARL2_ERR_HIP, "%s: the events measured no time", fn);
  *tflops = arl2::mfma_peak_flops(cus, iters) / ((double)ms * 1e-3) / 1e12;
  return ok();
}

}  // extern "C"
