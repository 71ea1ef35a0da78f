// kda_api.cpp -- the C ABI of libkda.so: argument validation, error codes,
// per-thread error text and dispatch to the kernel launchers.
//
// Every check happens before any HIP call, so a call that fails validation
// launches nothing and touches no device state (and can be made on a machine
// without a GPU).
#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "kda_internal.h"

namespace kda {

namespace {
thread_local char g_err[512] = "";

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_n(const void* p, unsigned n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }
bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool dtype_ok(int t) { return t == KDA_F32 || t == KDA_BF16; }
unsigned esize(int t) { return t == KDA_BF16 ? 2u : 4u; }

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

#define REQUIRE_PTR(p) \
  if ((p) == nullptr) return kda::fail(KDA_E_NULL, "%s is NULL", #p)
#define REQUIRE_A16(p) \
  if ((p) != nullptr && !kda::aligned16(p)) return kda::fail(KDA_E_ALIGN, "%s is not 16-byte aligned", #p)

int check_common(int B, int T, int H, int dk, int dv, int in_dtype, int out_dtype) {
  if (B < 1 || H < 1 || T < 0) return fail(KDA_E_SHAPE, "B=%d H=%d T=%d out of range", B, H, T);
  if (dk < 1 || dv < 1) return fail(KDA_E_SHAPE, "dk=%d dv=%d out of range", dk, dv);
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype))
    return fail(KDA_E_DTYPE, "in_dtype=%d out_dtype=%d not KDA_F32/KDA_BF16", in_dtype, out_dtype);
  if (!dim_ok(dk) || !dim_ok(dv) || dk != dv)
    return fail(KDA_E_UNSUPPORTED, "dk=%d dv=%d: head dims must be equal and in {16,32,64,128}", dk, dv);
  if ((long long)B * H > 0x7fffffffLL) return fail(KDA_E_SHAPE, "B*H=%lld too large", (long long)B * H);
  return KDA_OK;
}

// Workspace of kda_prefill_cp, in order: the segments' raw conv histories,
// then the final states from S = 0 (N), from S = I (P), the entering states
// (first the identity), and the segment prefills' own workspace.
size_t round256(size_t x) { return (x + 255) / 256 * 256; }

struct CpLayout {
  size_t n, p, s, pf, total;
};

kda_prefill_args cp_segment_args(const kda_prefill_cp_args& c) {
  kda_prefill_args s = c.prefill;
  s.B = c.prefill.B * c.segments;
  s.T = c.prefill.T / c.segments;
  s.workspace = nullptr;
  s.workspace_bytes = 0;
  return s;
}

CpLayout cp_layout(const kda_prefill_cp_args& c) {
  const kda_prefill_args& a = c.prefill;
  const size_t bs = (size_t)a.B * c.segments;
  const size_t cch = (size_t)a.H * (2 * a.dk + a.dv);
  const size_t states = round256(bs * a.H * a.dk * a.dv * sizeof(float));
  CpLayout l{};
  l.n = round256(bs * 3 * cch * esize(a.in_dtype));
  l.p = l.n + states;
  l.s = l.p + states;
  l.pf = l.s + states;
  l.total = l.pf + prefill_split_workspace_bytes(cp_segment_args(c));
  return l;
}

int check_decay(int form, const float* A) {
  if (form != KDA_DECAY_DIRECT && form != KDA_DECAY_K3)
    return fail(KDA_E_UNSUPPORTED, "decay_form=%d not KDA_DECAY_DIRECT/KDA_DECAY_K3", form);
  if (form == KDA_DECAY_K3) {
    if (A == nullptr) return fail(KDA_E_NULL, "A is NULL (decay_form KDA_DECAY_K3)");
    if (!aligned16(A)) return fail(KDA_E_ALIGN, "A is not 16-byte aligned");
  }
  return KDA_OK;
}
}  // namespace

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}

// ---- streams and events kept between calls -------------------------------------
// Handles are heap-held in a leaked registry, so they are still reachable when
// the exit handler runs, whatever order static objects are destroyed in.
namespace {
struct Kept {
  std::mutex mu;
  std::vector<hipStream_t> streams;
  std::vector<hipEvent_t> events;
};
Kept& kept() {
  static Kept* k = new Kept;
  return *k;
}
std::atomic<unsigned> g_generation{1};
std::once_flag g_at_exit;

// Destroy everything registered; the first failure is returned (the rest are
// still destroyed).
hipError_t release_all() {
  Kept& k = kept();
  std::lock_guard<std::mutex> lock(k.mu);
  g_generation.fetch_add(1);
  hipError_t first = hipSuccess;
  for (hipStream_t s : k.streams) {
    hipError_t e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipStreamDestroy(s);
    if (first == hipSuccess) first = e;
  }
  for (hipEvent_t ev : k.events) {
    const hipError_t e = hipEventDestroy(ev);
    if (first == hipSuccess) first = e;
  }
  k.streams.clear();
  k.events.clear();
  return first;
}

// Registered with atexit() when the first handle is kept, which is after the
// HIP runtime (and any tool loaded with it) registered its own teardown, so
// this runs before that teardown.
void release_at_exit() { (void)release_all(); }

void arm_exit_release() {
  std::call_once(g_at_exit, [] { std::atexit(release_at_exit); });
}
}  // namespace

void keep(hipStream_t s) {
  arm_exit_release();
  Kept& k = kept();
  std::lock_guard<std::mutex> lock(k.mu);
  k.streams.push_back(s);
}

void keep(hipEvent_t e) {
  arm_exit_release();
  Kept& k = kept();
  std::lock_guard<std::mutex> lock(k.mu);
  k.events.push_back(e);
}

unsigned release_generation() { return g_generation.load(); }

}  // namespace kda

using kda::fail;

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

int kda_wait_timeouts(unsigned* count) {
  if (count == nullptr) return fail(KDA_E_NULL, "wait_timeouts: count is NULL");
  return kda::wait_timeouts(count);
}

int kda_debug_pipeline(unsigned wait_limit_us, int withhold_slab) {
  if (withhold_slab < -1) return fail(KDA_E_SHAPE, "debug_pipeline: withhold_slab %d < -1", withhold_slab);
  kda::debug_pipeline(wait_limit_us, withhold_slab);
  return KDA_OK;
}

int kda_release(void) {
  const hipError_t e = kda::release_all();
  if (e != hipSuccess) return fail(KDA_E_HIP, "release: %s", hipGetErrorString(e));
  return KDA_OK;
}

const char* kda_last_error(void) { return kda::g_err; }

const char* kda_status_string(int code) {
  switch (code) {
    case KDA_OK: return "ok";
    case KDA_E_NULL: return "a required pointer is NULL";
    case KDA_E_SHAPE: return "a size is out of range";
    case KDA_E_DTYPE: return "unknown dtype";
    case KDA_E_ALIGN: return "a pointer is not 16-byte aligned";
    case KDA_E_UNSUPPORTED: return "unsupported head dim or chunk size";
    case KDA_E_WORKSPACE: return "workspace too small";
    case KDA_E_HIP: return "HIP runtime error";
    default: return "unknown status code";
  }
}

size_t kda_prefill_workspace_bytes(const kda_prefill_args* a) {
  if (a == nullptr) return 0;
  if (kda::check_common(a->B, a->T, a->H, a->dk, a->dv, a->in_dtype, a->out_dtype) != KDA_OK) return 0;
  return kda::prefill_split_workspace_bytes(*a);
}

size_t kda_prefill_workspace_min_bytes(const kda_prefill_args* a) {
  if (a == nullptr) return 0;
  if (kda::check_common(a->B, a->T, a->H, a->dk, a->dv, a->in_dtype, a->out_dtype) != KDA_OK) return 0;
  return kda::prefill_split_workspace_min_bytes(*a);
}

namespace kda {
namespace {
// Argument checks of kda_prefill and kda_prefill_noalloc (all but the workspace).
int check_prefill(const kda_prefill_args* a) {
  REQUIRE_PTR(a);
  int rc = kda::check_common(a->B, a->T, a->H, a->dk, a->dv, a->in_dtype, a->out_dtype);
  if (rc != KDA_OK) return rc;
  if (a->chunk != 16 && a->chunk != 32 && a->chunk != 64)
    return fail(KDA_E_UNSUPPORTED, "chunk=%d not in {16,32,64}", a->chunk);
  rc = kda::check_decay(a->decay_form, a->A);
  if (rc != KDA_OK) return rc;
  if (a->T > 0) {
    REQUIRE_PTR(a->q); REQUIRE_PTR(a->k); REQUIRE_PTR(a->v); REQUIRE_PTR(a->conv_w);
    REQUIRE_PTR(a->g); REQUIRE_PTR(a->beta); REQUIRE_PTR(a->gate); REQUIRE_PTR(a->o);
  }
  REQUIRE_A16(a->q); REQUIRE_A16(a->k); REQUIRE_A16(a->v); REQUIRE_A16(a->conv_w);
  REQUIRE_A16(a->g); REQUIRE_A16(a->gate); REQUIRE_A16(a->o); REQUIRE_A16(a->S0);
  REQUIRE_A16(a->S_T); REQUIRE_A16(a->conv_in); REQUIRE_A16(a->conv_out);
  if (a->beta != nullptr && !kda::aligned_n(a->beta, kda::esize(a->in_dtype)))
    return fail(KDA_E_ALIGN, "beta is not aligned to its element size");
  return KDA_OK;
}
}  // namespace
}  // namespace kda

int kda_prefill(const kda_prefill_args* a, void* stream) {
  kda::g_err[0] = '\0';
  const int rc = kda::check_prefill(a);
  if (rc != KDA_OK) return rc;
  REQUIRE_A16(a->workspace);
  if (a->workspace != nullptr && a->workspace_bytes < kda_prefill_workspace_min_bytes(a))
    return fail(KDA_E_WORKSPACE, "workspace %zu bytes < %zu", a->workspace_bytes,
                kda_prefill_workspace_min_bytes(a));
  if (a->T == 0 && a->S_T == nullptr && a->conv_out == nullptr) return KDA_OK;
  return kda::launch_prefill(*a, reinterpret_cast<hipStream_t>(stream));
}

int kda_prefill_noalloc(const kda_prefill_args* a, void* stream) {
  kda::g_err[0] = '\0';
  const int rc = kda::check_prefill(a);
  if (rc != KDA_OK) return rc;
  if (a->T == 0 && a->S_T == nullptr && a->conv_out == nullptr) return KDA_OK;
  return kda::launch_prefill_noalloc(*a, reinterpret_cast<hipStream_t>(stream));
}

size_t kda_cp_rank_workspace_bytes(const kda_prefill_args* a) {
  if (a == nullptr) return 0;
  if (kda::check_common(a->B, a->T, a->H, a->dk, a->dv, a->in_dtype, a->out_dtype) != KDA_OK) return 0;
  if (a->chunk != 16 && a->chunk != 32 && a->chunk != 64) return 0;
  const size_t split = kda::cp_rank_split_bytes(*a);
  if (split > 0) return split;
  // other sizes: three single-kernel prefills; the workspace holds the identity
  return kda::round256((size_t)a->B * a->H * a->dk * a->dv * sizeof(float));
}

int kda_cp_fragments(const kda_prefill_args* a, float* N, float* P, void* stream) {
  kda::g_err[0] = '\0';
  int rc = kda::check_prefill(a);
  if (rc != KDA_OK) return rc;
  REQUIRE_PTR(N); REQUIRE_PTR(P); REQUIRE_A16(N); REQUIRE_A16(P);
  REQUIRE_PTR(a->workspace); REQUIRE_A16(a->workspace);
  const size_t need = kda_cp_rank_workspace_bytes(a);
  if (a->workspace_bytes < need) return fail(KDA_E_WORKSPACE, "workspace %zu bytes < %zu", a->workspace_bytes, need);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t nstate = (size_t)a->B * a->H;
  if (a->T > 0 && kda::cp_rank_split_bytes(*a) > 0) return kda::launch_cp_fragments_split(*a, N, P, s);
  // T = 0 or sizes without the two-kernel path: plain prefills from S = 0 and
  // S = I (o serves as scratch; the finishing call overwrites it)
  float* eye = static_cast<float*>(a->workspace);
  rc = kda::launch_cp_identity(eye, nstate, a->dk, s);
  if (rc != KDA_OK) return rc;
  kda_prefill_args z = *a;
  z.workspace = nullptr;
  z.workspace_bytes = 0;
  z.conv_out = nullptr;
  z.S0 = nullptr;
  z.S_T = N;
  rc = kda_prefill(&z, stream);
  if (rc != KDA_OK) return rc;
  z.S0 = eye;
  z.S_T = P;
  return kda_prefill(&z, stream);
}

int kda_cp_finish(const kda_prefill_args* a, void* stream) {
  kda::g_err[0] = '\0';
  const int rc = kda::check_prefill(a);
  if (rc != KDA_OK) return rc;
  REQUIRE_PTR(a->workspace); REQUIRE_A16(a->workspace);
  const size_t need = kda_cp_rank_workspace_bytes(a);
  if (a->workspace_bytes < need) return fail(KDA_E_WORKSPACE, "workspace %zu bytes < %zu", a->workspace_bytes, need);
  if (a->T > 0 && kda::cp_rank_split_bytes(*a) > 0)
    return kda::launch_cp_finish_split(*a, reinterpret_cast<hipStream_t>(stream));
  kda_prefill_args z = *a;
  z.workspace = nullptr;
  z.workspace_bytes = 0;
  return kda_prefill(&z, stream);
}

int kda_cp_compose(const kda_cp_compose_args* a, void* stream) {
  kda::g_err[0] = '\0';
  REQUIRE_PTR(a);
  if (a->B < 1 || a->R < 1 || a->H < 1) return fail(KDA_E_SHAPE, "B=%d R=%d H=%d out of range", a->B, a->R, a->H);
  if ((long long)a->B * a->R * a->H > 0x7fffffffLL) return fail(KDA_E_SHAPE, "B*R*H too large");
  if (!kda::dim_ok(a->d)) return fail(KDA_E_UNSUPPORTED, "d=%d not in {16,32,64,128}", a->d);
  REQUIRE_PTR(a->N); REQUIRE_PTR(a->P); REQUIRE_PTR(a->S_start);
  REQUIRE_A16(a->N); REQUIRE_A16(a->P); REQUIRE_A16(a->S0); REQUIRE_A16(a->S_start); REQUIRE_A16(a->S_T);
  return kda::launch_cp_compose(*a, reinterpret_cast<hipStream_t>(stream));
}

size_t kda_prefill_cp_workspace_bytes(const kda_prefill_cp_args* c) {
  if (c == nullptr) return 0;
  const kda_prefill_args& a = c->prefill;
  if (kda::check_common(a.B, a.T, a.H, a.dk, a.dv, a.in_dtype, a.out_dtype) != KDA_OK) return 0;
  if (a.chunk != 16 && a.chunk != 32 && a.chunk != 64) return 0;
  if (c->segments < 1 || a.T % c->segments != 0 || a.T / c->segments < 3) return 0;
  if ((long long)a.B * c->segments * a.H > 0x7fffffffLL) return 0;
  return kda::cp_layout(*c).total;
}

int kda_prefill_cp(const kda_prefill_cp_args* c, void* stream) {
  kda::g_err[0] = '\0';
  REQUIRE_PTR(c);
  const kda_prefill_args& a = c->prefill;
  int rc = kda::check_common(a.B, a.T, a.H, a.dk, a.dv, a.in_dtype, a.out_dtype);
  if (rc != KDA_OK) return rc;
  if (a.chunk != 16 && a.chunk != 32 && a.chunk != 64)
    return fail(KDA_E_UNSUPPORTED, "chunk=%d not in {16,32,64}", a.chunk);
  rc = kda::check_decay(a.decay_form, a.A);
  if (rc != KDA_OK) return rc;
  const int R = c->segments;
  if (R < 1) return fail(KDA_E_SHAPE, "segments=%d < 1", R);
  if (a.T == 0) {  // nothing to split: the carry copies of kda_prefill
    kda_prefill_args z = a;
    z.workspace = nullptr;
    z.workspace_bytes = 0;
    return kda_prefill(&z, stream);
  }
  if (a.T % R != 0 || a.T / R < 3)
    return fail(KDA_E_SHAPE, "T=%d is not a multiple of segments=%d with at least 3 tokens each", a.T, R);
  if ((long long)a.B * R * a.H > 0x7fffffffLL) return fail(KDA_E_SHAPE, "B*segments*H too large");
  REQUIRE_PTR(a.q); REQUIRE_PTR(a.k); REQUIRE_PTR(a.v); REQUIRE_PTR(a.conv_w);
  REQUIRE_PTR(a.g); REQUIRE_PTR(a.beta); REQUIRE_PTR(a.gate); REQUIRE_PTR(a.o);
  REQUIRE_A16(a.q); REQUIRE_A16(a.k); REQUIRE_A16(a.v); REQUIRE_A16(a.conv_w);
  REQUIRE_A16(a.g); REQUIRE_A16(a.gate); REQUIRE_A16(a.o); REQUIRE_A16(a.S0);
  REQUIRE_A16(a.S_T); REQUIRE_A16(a.conv_in); REQUIRE_A16(a.conv_out);
  if (!kda::aligned_n(a.beta, kda::esize(a.in_dtype)))
    return fail(KDA_E_ALIGN, "beta is not aligned to its element size");
  if (c->workspace == nullptr) return fail(KDA_E_NULL, "workspace is NULL (kda_prefill_cp_workspace_bytes)");
  REQUIRE_A16(c->workspace);
  const kda::CpLayout l = kda::cp_layout(*c);
  if (c->workspace_bytes < l.total)
    return fail(KDA_E_WORKSPACE, "workspace %zu bytes < %zu", c->workspace_bytes, l.total);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  unsigned char* ws = static_cast<unsigned char*>(c->workspace);
  float* Nb = reinterpret_cast<float*>(ws + l.n);
  float* Pb = reinterpret_cast<float*>(ws + l.p);
  float* Sb = reinterpret_cast<float*>(ws + l.s);
  const int L = a.T / R;
  const size_t bs = (size_t)a.B * R;
  // 1. every segment's raw conv history
  rc = kda::launch_cp_history(a, R, 0, L, ws, s);
  if (rc != KDA_OK) return rc;
  // 2. the fragments: all segments from S = 0 (N) and from S = I (P)
  kda_prefill_args sa = kda::cp_segment_args(*c);
  sa.conv_in = ws;
  sa.conv_out = nullptr;
  if (l.total > l.pf) {
    sa.workspace = ws + l.pf;
    sa.workspace_bytes = l.total - l.pf;
  }
  sa.S0 = nullptr;
  sa.S_T = Nb;
  rc = kda_prefill(&sa, stream);
  if (rc != KDA_OK) return rc;
  rc = kda::launch_cp_identity(Sb, bs * a.H, a.dk, s);
  if (rc != KDA_OK) return rc;
  sa.S0 = Sb;
  sa.S_T = Pb;
  rc = kda_prefill(&sa, stream);
  if (rc != KDA_OK) return rc;
  // 3. the entering state of every segment
  const kda_cp_compose_args ca{a.B, R, a.H, a.dk, Nb, Pb, a.S0, Sb, nullptr};
  rc = kda::launch_cp_compose(ca, s);
  if (rc != KDA_OK) return rc;
  // 4. every segment from its entering state; the last segment's final state
  sa.S0 = Sb;
  sa.S_T = a.S_T != nullptr ? Pb : nullptr;
  rc = kda_prefill(&sa, stream);
  if (rc != KDA_OK) return rc;
  if (a.S_T != nullptr) {
    const size_t per = (size_t)a.H * a.dk * a.dv;
    for (int b = 0; b < a.B; ++b) {
      const hipError_t e = hipMemcpyAsync(a.S_T + (size_t)b * per, Pb + ((size_t)b * R + R - 1) * per,
                                          per * sizeof(float), hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return fail(KDA_E_HIP, "state copy failed: %s", hipGetErrorString(e));
    }
  }
  if (a.conv_out != nullptr) return kda::launch_cp_history(a, 1, R, L, a.conv_out, s);
  return KDA_OK;
}

size_t kda_prefill_backward_workspace_bytes(const kda_prefill_backward_args* a) {
  if (a == nullptr) return 0;
  if (kda::check_common(a->B, a->T, a->H, a->dk, a->dv, a->in_dtype, KDA_F32) != KDA_OK) return 0;
  return kda::prefill_backward_workspace_bytes(*a);
}

int kda_prefill_backward(const kda_prefill_backward_args* a, void* stream) {
  kda::g_err[0] = '\0';
  REQUIRE_PTR(a);
  int rc = kda::check_common(a->B, a->T, a->H, a->dk, a->dv, a->in_dtype, KDA_F32);
  if (rc != KDA_OK) return rc;
  if (a->decay_form != KDA_DECAY_DIRECT)
    return fail(KDA_E_UNSUPPORTED, "backward: decay_form=%d; only KDA_DECAY_DIRECT", a->decay_form);
  if ((long long)a->B * a->T * a->H > 0x7fffffffLL) return fail(KDA_E_SHAPE, "B*T*H too large");
  if (a->T > 0) {
    REQUIRE_PTR(a->q); REQUIRE_PTR(a->k); REQUIRE_PTR(a->v); REQUIRE_PTR(a->conv_w);
    REQUIRE_PTR(a->g); REQUIRE_PTR(a->beta); REQUIRE_PTR(a->gate); REQUIRE_PTR(a->grad_o);
    REQUIRE_PTR(a->grad_q); REQUIRE_PTR(a->grad_k); REQUIRE_PTR(a->grad_v); REQUIRE_PTR(a->grad_g);
    REQUIRE_PTR(a->grad_beta); REQUIRE_PTR(a->grad_gate);
  }
  REQUIRE_A16(a->q); REQUIRE_A16(a->k); REQUIRE_A16(a->v); REQUIRE_A16(a->conv_w);
  REQUIRE_A16(a->g); REQUIRE_A16(a->gate); REQUIRE_A16(a->S0); REQUIRE_A16(a->conv_in);
  REQUIRE_A16(a->grad_o); REQUIRE_A16(a->grad_S_T); REQUIRE_A16(a->grad_conv_out);
  REQUIRE_A16(a->grad_q); REQUIRE_A16(a->grad_k);
  REQUIRE_A16(a->grad_v); REQUIRE_A16(a->grad_g); REQUIRE_A16(a->grad_gate); REQUIRE_A16(a->grad_S0);
  REQUIRE_A16(a->grad_conv_in);
  if (a->beta != nullptr && !kda::aligned_n(a->beta, kda::esize(a->in_dtype)))
    return fail(KDA_E_ALIGN, "beta is not aligned to its element size");
  if (a->grad_beta != nullptr && !kda::aligned_n(a->grad_beta, 4))
    return fail(KDA_E_ALIGN, "grad_beta is not 4-byte aligned");
  if (a->workspace == nullptr) return fail(KDA_E_NULL, "workspace is NULL (kda_prefill_backward_workspace_bytes)");
  REQUIRE_A16(a->workspace);
  const size_t need = kda::prefill_backward_workspace_bytes(*a);
  if (a->workspace_bytes < need) return fail(KDA_E_WORKSPACE, "workspace %zu bytes < %zu", a->workspace_bytes, need);
  return kda::launch_prefill_backward(*a, reinterpret_cast<hipStream_t>(stream));
}

int kda_decode_step(const kda_decode_args* a, void* stream) {
  kda::g_err[0] = '\0';
  REQUIRE_PTR(a);
  int rc = kda::check_common(a->N, 1, a->H, a->dk, a->dv, a->in_dtype, a->out_dtype);
  if (rc != KDA_OK) return rc;
  rc = kda::check_decay(a->decay_form, a->A);
  if (rc != KDA_OK) return rc;
  REQUIRE_PTR(a->q); REQUIRE_PTR(a->k); REQUIRE_PTR(a->v); REQUIRE_PTR(a->conv_w);
  REQUIRE_PTR(a->g); REQUIRE_PTR(a->beta); REQUIRE_PTR(a->gate); REQUIRE_PTR(a->S);
  REQUIRE_PTR(a->conv_state); REQUIRE_PTR(a->o);
  REQUIRE_A16(a->q); REQUIRE_A16(a->k); REQUIRE_A16(a->v); REQUIRE_A16(a->conv_w);
  REQUIRE_A16(a->g); REQUIRE_A16(a->gate); REQUIRE_A16(a->S); REQUIRE_A16(a->conv_state);
  REQUIRE_A16(a->o);
  if (!kda::aligned_n(a->beta, kda::esize(a->in_dtype)))
    return fail(KDA_E_ALIGN, "beta is not aligned to its element size");
  return kda::launch_decode(*a, reinterpret_cast<hipStream_t>(stream));
}

int kda_decode_multi(const kda_decode_multi_args* a, void* stream) {
  kda::g_err[0] = '\0';
  REQUIRE_PTR(a);
  int rc = kda::check_common(a->N, 1, a->H, a->dk, a->dv, a->in_dtype, a->out_dtype);
  if (rc != KDA_OK) return rc;
  if (a->M < 1 || a->M > KDA_MAX_DECODE_TOKENS)
    return fail(KDA_E_SHAPE, "M=%d not in [1, %d]", a->M, KDA_MAX_DECODE_TOKENS);
  if ((long long)a->N * a->M * a->H > 0x7fffffffLL)
    return fail(KDA_E_SHAPE, "N*M*H too large");
  rc = kda::check_decay(a->decay_form, a->A);
  if (rc != KDA_OK) return rc;
  REQUIRE_PTR(a->q); REQUIRE_PTR(a->k); REQUIRE_PTR(a->v); REQUIRE_PTR(a->conv_w);
  REQUIRE_PTR(a->g); REQUIRE_PTR(a->beta); REQUIRE_PTR(a->gate); REQUIRE_PTR(a->S);
  REQUIRE_PTR(a->conv_state); REQUIRE_PTR(a->o);
  REQUIRE_A16(a->q); REQUIRE_A16(a->k); REQUIRE_A16(a->v); REQUIRE_A16(a->conv_w);
  REQUIRE_A16(a->g); REQUIRE_A16(a->gate); REQUIRE_A16(a->S); REQUIRE_A16(a->conv_state);
  REQUIRE_A16(a->o);
  if (!kda::aligned_n(a->beta, kda::esize(a->in_dtype)))
    return fail(KDA_E_ALIGN, "beta is not aligned to its element size");
  if (a->accept != nullptr && !kda::aligned_n(a->accept, 4))
    return fail(KDA_E_ALIGN, "accept is not 4-byte aligned");
  return kda::launch_decode_multi(*a, reinterpret_cast<hipStream_t>(stream));
}

int kda_prep(const kda_prep_args* a, void* stream) {
  kda::g_err[0] = '\0';
  REQUIRE_PTR(a);
  int rc = kda::check_common(a->B, a->T, a->H, a->dk, a->dv, a->in_dtype, KDA_F32);
  if (rc != KDA_OK) return rc;
  rc = kda::check_decay(a->decay_form, a->A);
  if (rc != KDA_OK) return rc;
  if (a->chunk != 16 && a->chunk != 32 && a->chunk != 64)
    return fail(KDA_E_UNSUPPORTED, "chunk=%d not in {16,32,64}", a->chunk);
  if (a->T == 0) return KDA_OK;
  REQUIRE_PTR(a->q); REQUIRE_PTR(a->k); REQUIRE_PTR(a->v); REQUIRE_PTR(a->conv_w);
  REQUIRE_PTR(a->g); REQUIRE_PTR(a->q_out); REQUIRE_PTR(a->k_out); REQUIRE_PTR(a->v_out);
  REQUIRE_PTR(a->G_out);
  REQUIRE_A16(a->q); REQUIRE_A16(a->k); REQUIRE_A16(a->v); REQUIRE_A16(a->conv_w);
  REQUIRE_A16(a->g); REQUIRE_A16(a->conv_in); REQUIRE_A16(a->q_out); REQUIRE_A16(a->k_out);
  REQUIRE_A16(a->v_out); REQUIRE_A16(a->G_out);
  const long long nchunks = (a->T + a->chunk - 1) / a->chunk;
  if ((long long)a->B * a->H * nchunks > 0xffffffffLL)
    return fail(KDA_E_SHAPE, "B*H*chunks too large for one launch");
  return kda::launch_prep(*a, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
