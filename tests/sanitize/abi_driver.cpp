// Host-side driver for the sanitizer build of the C ABI (kda_api.cpp built
// with AddressSanitizer and UndefinedBehaviorSanitizer): every export's
// argument validation, the workspace queries over a range of shapes, the
// status strings and the release path.  No call here passes validation into
// a launch, so it runs without a GPU.  Exit status 0 when every result is the
// expected one.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "kda.h"

static int g_fail = 0;
#define EXPECT(cond)                                                 \
  do {                                                               \
    if (!(cond)) {                                                   \
      std::fprintf(stderr, "line %d: %s failed\n", __LINE__, #cond); \
      ++g_fail;                                                      \
    }                                                                \
  } while (0)

// aligned stand-in device addresses (never dereferenced on the host)
static void* fake(uintptr_t k) { return reinterpret_cast<void*>(uintptr_t(1) << 20 | (k << 12)); }

static kda_prefill_args prefill_base(int B, int T, int H, int d, int chunk, int dt) {
  kda_prefill_args a;
  std::memset(&a, 0, sizeof a);
  a.B = B; a.T = T; a.H = H; a.dk = d; a.dv = d; a.chunk = chunk; a.in_dtype = dt; a.out_dtype = KDA_F32;
  a.q = fake(1); a.k = fake(2); a.v = fake(3); a.conv_w = static_cast<const float*>(fake(4));
  a.g = fake(5); a.beta = fake(6); a.gate = fake(7); a.o = fake(8);
  return a;
}

int main() {
  // status strings of every code and beyond
  for (int c = -12; c <= 2; ++c) EXPECT(kda_status_string(c) != nullptr && std::strlen(kda_status_string(c)) > 0);
  EXPECT(kda_abi_version() == KDA_ABI_VERSION);

  // ---- kda_prefill / kda_prefill_noalloc validation -----------------------------
  EXPECT(kda_prefill(nullptr, nullptr) == KDA_E_NULL);
  EXPECT(kda_prefill_noalloc(nullptr, nullptr) == KDA_E_NULL);
  {
    kda_prefill_args a = prefill_base(0, 10, 2, 64, 64, KDA_BF16);
    EXPECT(kda_prefill(&a, nullptr) == KDA_E_SHAPE);
    a = prefill_base(1, -1, 2, 64, 64, KDA_BF16);
    EXPECT(kda_prefill(&a, nullptr) == KDA_E_SHAPE);
    a = prefill_base(1, 10, 2, 64, 64, 7);
    EXPECT(kda_prefill(&a, nullptr) == KDA_E_DTYPE);
    a = prefill_base(1, 10, 2, 48, 64, KDA_BF16);
    EXPECT(kda_prefill(&a, nullptr) == KDA_E_UNSUPPORTED);
    a = prefill_base(1, 10, 2, 64, 48, KDA_BF16);
    EXPECT(kda_prefill(&a, nullptr) == KDA_E_UNSUPPORTED);
    a = prefill_base(1, 10, 2, 64, 64, KDA_BF16);
    a.q = nullptr;
    EXPECT(kda_prefill(&a, nullptr) == KDA_E_NULL);
    EXPECT(std::strstr(kda_last_error(), "q") != nullptr);
    a = prefill_base(1, 10, 2, 64, 64, KDA_BF16);
    a.k = static_cast<const char*>(a.k) + 2;
    EXPECT(kda_prefill(&a, nullptr) == KDA_E_ALIGN);
    a = prefill_base(1, 10, 2, 64, 64, KDA_BF16);
    a.decay_form = 5;
    EXPECT(kda_prefill(&a, nullptr) == KDA_E_UNSUPPORTED);
    a.decay_form = KDA_DECAY_K3;  // A missing
    EXPECT(kda_prefill(&a, nullptr) == KDA_E_NULL);
    a = prefill_base(1, 1000, 2, 128, 64, KDA_BF16);
    a.workspace = fake(9);
    a.workspace_bytes = 16;  // below the minimum
    EXPECT(kda_prefill(&a, nullptr) == KDA_E_WORKSPACE);
    // no-allocation entry: more heads than its scratch holds
    a = prefill_base(1, 128, 1025, 128, 64, KDA_BF16);
    EXPECT(kda_prefill_noalloc(&a, nullptr) == KDA_E_WORKSPACE);
    EXPECT(std::strstr(kda_last_error(), "scratch") != nullptr);
    // T = 0 with nothing to write: a valid no-op
    a = prefill_base(1, 0, 2, 64, 64, KDA_BF16);
    EXPECT(kda_prefill(&a, nullptr) == KDA_OK);
    EXPECT(kda_prefill_noalloc(&a, nullptr) == KDA_OK);
  }
  // workspace queries over shapes (two-kernel shapes report > 0, others 0)
  {
    const int Ts[] = {1, 63, 64, 65, 4096, 65536, 1 << 20};
    const int Hs[] = {1, 32, 96, 128, 200};
    size_t total = 0;
    for (int T : Ts)
      for (int H : Hs) {
        kda_prefill_args a = prefill_base(1, T, H, 128, 64, KDA_BF16);
        const size_t pref = kda_prefill_workspace_bytes(&a), mn = kda_prefill_workspace_min_bytes(&a);
        EXPECT(pref >= mn && mn > 0);
        total += pref;
        a.in_dtype = KDA_F32;
        EXPECT(kda_prefill_workspace_bytes(&a) == 0);
        kda_prefill_cp_args c;
        std::memset(&c, 0, sizeof c);
        c.prefill = prefill_base(1, T, H, 128, 64, KDA_BF16);
        c.segments = 4;
        const size_t cw = kda_prefill_cp_workspace_bytes(&c);
        EXPECT(T % 4 != 0 || T / 4 < 3 ? cw == 0 : cw > 0);
      }
    EXPECT(total > 0);
    EXPECT(kda_prefill_workspace_bytes(nullptr) == 0);
    EXPECT(kda_prefill_cp_workspace_bytes(nullptr) == 0);
  }

  // ---- decode ---------------------------------------------------------------------
  {
    EXPECT(kda_decode_step(nullptr, nullptr) == KDA_E_NULL);
    kda_decode_args d;
    std::memset(&d, 0, sizeof d);
    d.N = 4; d.H = 2; d.dk = 128; d.dv = 128; d.in_dtype = KDA_BF16; d.out_dtype = KDA_F32;
    EXPECT(kda_decode_step(&d, nullptr) == KDA_E_NULL);  // no pointers
    d.q = fake(1); d.k = fake(2); d.v = fake(3); d.conv_w = static_cast<const float*>(fake(4));
    d.g = fake(5); d.beta = fake(6); d.gate = fake(7); d.S = static_cast<float*>(fake(8));
    d.conv_state = fake(9); d.o = fake(10);
    d.N = 0;
    EXPECT(kda_decode_step(&d, nullptr) == KDA_E_SHAPE);
    d.N = 4; d.dk = 100;
    EXPECT(kda_decode_step(&d, nullptr) == KDA_E_UNSUPPORTED);
    d.dk = 128; d.S = reinterpret_cast<float*>(static_cast<char*>(fake(8)) + 4);
    EXPECT(kda_decode_step(&d, nullptr) == KDA_E_ALIGN);

    EXPECT(kda_decode_multi(nullptr, nullptr) == KDA_E_NULL);
    kda_decode_multi_args m;
    std::memset(&m, 0, sizeof m);
    m.N = 4; m.M = KDA_MAX_DECODE_TOKENS + 1; m.H = 2; m.dk = 128; m.dv = 128; m.in_dtype = KDA_BF16;
    m.q = fake(1); m.k = fake(2); m.v = fake(3); m.conv_w = static_cast<const float*>(fake(4));
    m.g = fake(5); m.beta = fake(6); m.gate = fake(7); m.S = static_cast<float*>(fake(8));
    m.conv_state = fake(9); m.o = fake(10);
    EXPECT(kda_decode_multi(&m, nullptr) != KDA_OK);
    m.M = 0;
    EXPECT(kda_decode_multi(&m, nullptr) != KDA_OK);
  }

  // ---- prep, context parallel, composition ------------------------------------------
  {
    EXPECT(kda_prep(nullptr, nullptr) == KDA_E_NULL);
    kda_prep_args p;
    std::memset(&p, 0, sizeof p);
    p.B = 1; p.T = 10; p.H = 2; p.dk = 64; p.dv = 64; p.chunk = 48; p.in_dtype = KDA_BF16;
    EXPECT(kda_prep(&p, nullptr) != KDA_OK);

    EXPECT(kda_prefill_cp(nullptr, nullptr) == KDA_E_NULL);
    kda_prefill_cp_args c;
    std::memset(&c, 0, sizeof c);
    c.prefill = prefill_base(1, 1000, 2, 64, 64, KDA_BF16);
    c.segments = 3;  // 1000 not divisible
    EXPECT(kda_prefill_cp(&c, nullptr) != KDA_OK);
    c.segments = 0;
    EXPECT(kda_prefill_cp(&c, nullptr) != KDA_OK);

    EXPECT(kda_cp_compose(nullptr, nullptr) == KDA_E_NULL);
    kda_cp_compose_args k;
    std::memset(&k, 0, sizeof k);
    k.B = 1; k.R = 4; k.H = 2; k.d = 40;
    EXPECT(kda_cp_compose(&k, nullptr) == KDA_E_UNSUPPORTED);
    k.d = 64;
    EXPECT(kda_cp_compose(&k, nullptr) == KDA_E_NULL);
  }

  // ---- backward ------------------------------------------------------------------------
  {
    EXPECT(kda_prefill_backward(nullptr, nullptr) == KDA_E_NULL);
    EXPECT(kda_prefill_backward_workspace_bytes(nullptr) == 0);
    kda_prefill_backward_args b;
    std::memset(&b, 0, sizeof b);
    b.B = 1; b.T = 1100; b.H = 2; b.dk = 128; b.dv = 128; b.in_dtype = KDA_BF16;
    EXPECT(kda_prefill_backward_workspace_bytes(&b) > 0);
    EXPECT(kda_prefill_backward(&b, nullptr) == KDA_E_NULL);
    b.dk = 96;
    EXPECT(kda_prefill_backward_workspace_bytes(&b) == 0);
  }

  // nothing was created, so nothing is destroyed (no HIP call)
  EXPECT(kda_release() == KDA_OK);
  EXPECT(kda_release() == KDA_OK);

  if (g_fail == 0) std::printf("abi driver: all checks passed\n");
  return g_fail == 0 ? 0 : 1;
}
