// Host-only driver of the C-ABI validation layer (api.cpp + shapes.cpp over
// the HIP stub), built under the address/undefined-behaviour sanitizers and,
// separately, the thread sanitizer.  Each case calls an entry point and checks
// the documented status code, that a rejected call launches nothing, and, for
// accepted calls, the arguments handed to the launcher (strides, head
// mapping, workspace layout).  Exit status 0 iff every check holds.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <thread>

#include "diffattn.h"
#include "hip_stub.h"

static int g_fail = 0;
static int g_checks = 0;

#define CHECK(cond)                                                             \
    do {                                                                        \
        ++g_checks;                                                             \
        if (!(cond)) {                                                          \
            std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++g_fail;                                                           \
        }                                                                       \
    } while (0)

static void* dev(uintptr_t off) { return reinterpret_cast<void*>(STUB_DEV_LO + off); }
static void* host(uintptr_t off) { return reinterpret_cast<void*>((uintptr_t)0x10000 + off); }

constexpr int OK = DIFFATTN_OK, INV = DIFFATTN_ERR_INVALID_ARGUMENT, UNS = DIFFATTN_ERR_UNSUPPORTED,
              WSP = DIFFATTN_ERR_WORKSPACE;

// Rejected calls launch nothing and leave a message.
static void expect_reject(int got, int want) {
    CHECK(got == want);
    CHECK(std::strlen(diffattn_last_error()) > 0);
}

struct Prefill {
    void *q1 = dev(0), *q2 = dev(128), *k1 = dev(1 << 20), *k2 = dev((1 << 20) + 128),
         *v = dev(2 << 20), *out = dev(3 << 20), *lam = dev(4 << 20), *w = nullptr;
    int64_t ldq = 128, ldk = 128, ldv = 128;
    int dt = DIFFATTN_BF16;
    int B = 2, H = 3, N = 100, d = 64, dv = 128, causal = 1, rms = 1;
    float eps = 1e-5f, scale = 0.5f;
    int call() const {
        return diffattn_prefill(q1, q2, k1, k2, v, ldq, ldk, ldv, dt, B, H, N, d, dv, causal,
                                (const float*)lam, rms, eps, scale, (const float*)w, (float*)out,
                                nullptr);
    }
};

static void prefill_cases() {
    const int before = g_stub.launches;
    { Prefill p; p.q1 = nullptr; expect_reject(p.call(), INV); }
    { Prefill p; p.B = 0; expect_reject(p.call(), INV); }
    { Prefill p; p.N = -5; expect_reject(p.call(), INV); }
    { Prefill p; p.dt = 9; expect_reject(p.call(), INV); }
    { Prefill p; p.dt = -1; expect_reject(p.call(), INV); }
    { Prefill p; p.ldq = 63; expect_reject(p.call(), INV); }
    { Prefill p; p.ldk = 68; expect_reject(p.call(), INV); }          // 136 bytes: not 16-aligned
    { Prefill p; p.q2 = dev(130); expect_reject(p.call(), INV); }
    { Prefill p; p.lam = dev((4 << 20) + 2); expect_reject(p.call(), INV); }
    { Prefill p; p.eps = -1.f; expect_reject(p.call(), INV); }
    { Prefill p; p.eps = NAN; expect_reject(p.call(), INV); }
    { Prefill p; p.d = 48; expect_reject(p.call(), UNS); }
    { Prefill p; p.dv = 96; p.ldv = 96; expect_reject(p.call(), UNS); }
    { Prefill p; p.ldv = (int64_t)1 << 24; expect_reject(p.call(), UNS); }
    { Prefill p; p.ldk = (int64_t)1 << 40; expect_reject(p.call(), UNS); }
    { Prefill p; p.B = 1 << 20; p.H = 1 << 20; p.N = 2; expect_reject(p.call(), INV); }
    { Prefill p; p.v = host(0); expect_reject(p.call(), INV); }      // not device memory
    { Prefill p; p.w = host(0); expect_reject(p.call(), INV); }
    CHECK(g_stub.launches == before);

    // Accepted: packed V1 tensors, the launcher sees per-head strides.
    {
        Prefill p;
        CHECK(p.call() == OK);
        CHECK(std::strcmp(g_stub.last, "prefill_bf16") == 0);
        const diffattn::PrefillArgs& a = g_stub.prefill;
        CHECK(a.B == 2 && a.H == 3 && a.N == 100 && a.d == 64 && a.dv == 128);
        CHECK(a.hs.qb == 3 * 100 * 128 && a.hs.qh == 100 * 128);
        CHECK(a.hs.kb == 3 * 100 * 128 && a.hs.kh == 100 * 128);
        CHECK(a.hs.vb == 3 * 100 * 128 && a.hs.vh == 100 * 128 && a.hs.kv_group == 1);
        CHECK(a.rmsnorm == 1 && a.norm_scale == 0.5f && a.norm_weight == nullptr);
    }
    {
        Prefill p;   // the largest bf16 token stride the kernels address
        p.ldq = p.ldk = p.ldv = ((int64_t)1 << 24) - 8;
        CHECK(p.call() == OK);
    }
    {
        Prefill p;   // fp32 takes any stride; the norm is dropped when off
        p.dt = DIFFATTN_FP32;
        p.ldq = p.ldk = p.ldv = (int64_t)1 << 24;
        p.rms = 0;
        p.w = dev(5 << 20);
        CHECK(p.call() == OK);
        CHECK(std::strcmp(g_stub.last, "prefill_f32") == 0);
        CHECK(g_stub.prefill.norm_weight == nullptr && g_stub.prefill.rmsnorm == 0);
    }
}

static void prefill_v2_cases() {
    void *q = dev(0), *k = dev(1 << 24), *v = dev(2 << 24), *lam = dev(3 << 24), *out = dev(4 << 24);
    auto call = [&](int dt, int B, int Hq, int Hkv, int N, int D) {
        return diffattn_prefill_v2(q, k, v, dt, B, Hq, Hkv, N, D, 1, (const float*)lam,
                                   (float*)out, nullptr);
    };
    const int before = g_stub.launches;
    expect_reject(call(DIFFATTN_BF16, 1, 6, 2, 64, 128), INV);     // Hq not a multiple of 2 Hkv
    expect_reject(call(DIFFATTN_BF16, 1, 8, 0, 64, 128), INV);
    expect_reject(call(DIFFATTN_BF16, 1, 8, 2, 64, 100), INV);     // 200-byte rows
    expect_reject(call(DIFFATTN_BF16, 1, 8, 2, 64, 32), UNS);
    expect_reject(call(7, 1, 8, 2, 64, 128), INV);
    CHECK(g_stub.launches == before);
    CHECK(call(DIFFATTN_BF16, 2, 32, 8, 1000, 128) == OK);
    const diffattn::PrefillArgs& a = g_stub.prefill;
    const int64_t ND = 1000 * 128;
    CHECK(a.H == 16 && a.d == 128 && a.dv == 128 && a.ldq == 128);
    CHECK((const char*)a.q2 - (const char*)a.q1 == ND * 2);
    CHECK(a.k1 == a.k2);
    CHECK(a.hs.qb == 32 * ND && a.hs.qh == 2 * ND && a.hs.kb == 8 * ND && a.hs.kh == ND);
    CHECK(a.hs.kv_group == 2);
}

static void decode_cases() {
    void *q = dev(0), *k = dev(1 << 24), *v = dev(2 << 24), *lens = dev(3 << 24), *lam = dev(4 << 24),
         *out = dev(5 << 24), *ws = dev(6 << 24);
    const int B = 4, Hq = 32, Hkv = 8, D = 128, L = 70000;
    const size_t need = diffattn_decode_workspace_bytes(B, Hq, Hkv, D, L);
    const size_t pieces = (L + 4095) / 4096 + 1;
    CHECK(need == (B * Hq * pieces * 130 + (size_t)B * Hq) * 4);
    CHECK(diffattn_decode_workspace_bytes(0, Hq, Hkv, D, L) == 0);
    auto call = [&](void* w, size_t bytes, int hq, int hkv, int d, int ml) {
        return diffattn_decode(q, k, v, (const int32_t*)lens, B, hq, hkv, d, ml, (const float*)lam,
                               w, bytes, (float*)out, nullptr);
    };
    const int before = g_stub.launches;
    expect_reject(call(ws, need, 30, 8, 128, L), INV);
    expect_reject(call(ws, need, Hq, Hkv, 64, L), UNS);
    expect_reject(call(ws, need, 64, 2, 128, L), UNS);              // 32 query heads per KV head
    expect_reject(call(ws, need - 1, Hq, Hkv, D, L), WSP);
    expect_reject(call(nullptr, need, Hq, Hkv, D, L), WSP);
    expect_reject(call(dev((6 << 24) + 16), need, Hq, Hkv, D, L), INV);   // not 256-aligned
    expect_reject(call(host(0), need, Hq, Hkv, D, L), INV);
    CHECK(g_stub.launches == before);
    CHECK(call(ws, need, Hq, Hkv, D, L) == OK);
    const diffattn::DecodeArgs& a = g_stub.decode;
    CHECK(a.B == B && a.Hq == Hq && a.Hkv == Hkv && a.D == D && a.max_len == L && a.qhalf == 0);

    // Plain single-map decode: Hq a multiple of Hkv, no lambda.
    auto plain = [&](int hq, int hkv, size_t bytes) {
        return diffattn_attention_decode(q, k, v, (const int32_t*)lens, B, hq, hkv, D, L, ws, bytes,
                                         (float*)out, nullptr);
    };
    const size_t need16 = diffattn_decode_workspace_bytes(B, 16, Hkv, D, L);
    CHECK(plain(16, Hkv, need16) == OK);
    CHECK(g_stub.decode.single == 1 && g_stub.decode.Hq == 16 && g_stub.decode.lambda == nullptr);
    CHECK(plain(8, 8, diffattn_decode_workspace_bytes(B, 8, 8, D, L)) == OK);    // one head per KV head
    const int before3 = g_stub.launches;
    expect_reject(plain(12, Hkv, need16), INV);
    expect_reject(plain(16, Hkv, need16 - 4), WSP);
    expect_reject(plain(Hkv * 17, Hkv, 1u << 30), UNS);
    CHECK(g_stub.launches == before3);

    // Allocation-free variant: the same checks, the fixed scratch bounds the sizes.
    auto noalloc = [&](int b, int ml) {
        return diffattn_decode_noalloc(q, k, v, (const int32_t*)lens, b, Hq, Hkv, D, ml,
                                       (const float*)lam, (float*)out, nullptr);
    };
    CHECK(noalloc(B, L) == OK);
    CHECK(std::strcmp(g_stub.last, "decode_noalloc") == 0 && g_stub.decode.workspace == nullptr);
    CHECK(diffattn_decode_workspace_bytes(B, Hq, Hkv, D, L) <= DIFFATTN_DECODE_SCRATCH_BYTES);
    const int before2 = g_stub.launches;
    CHECK(diffattn_decode_workspace_bytes(64, Hq, Hkv, D, 1 << 20) > DIFFATTN_DECODE_SCRATCH_BYTES);
    expect_reject(noalloc(64, 1 << 20), WSP);
    CHECK(std::strstr(diffattn_last_error(), "scratch") != nullptr);
    expect_reject(diffattn_decode_noalloc(q, k, v, (const int32_t*)lens, B, 30, Hkv, D, L,
                                          (const float*)lam, (float*)out, nullptr), INV);
    expect_reject(diffattn_decode_noalloc(q, k, v, (const int32_t*)lens, B, Hq, Hkv, D, L,
                                          (const float*)lam, (float*)host(0), nullptr), INV);
    CHECK(g_stub.launches == before2);

    // V1 layout: two query columns per head over its own rows.
    const size_t need1 = diffattn_decode_v1_workspace_bytes(B, 16, L);
    CHECK(need1 == diffattn_decode_workspace_bytes(B, 32, 16, 128, L));
    CHECK(diffattn_decode_v1(q, k, v, (const int32_t*)lens, B, 16, 64, 128, L, (const float*)lam,
                             1, 1e-5f, 0.25f, nullptr, ws, need1, (float*)out, nullptr) == OK);
    CHECK(g_stub.decode.Hq == 32 && g_stub.decode.Hkv == 16 && g_stub.decode.D == 128 &&
          g_stub.decode.qhalf == 64 && g_stub.decode.norm_scale == 0.25f);
    expect_reject(diffattn_decode_v1(q, k, v, (const int32_t*)lens, B, 16, 32, 128, L,
                                     (const float*)lam, 1, 1e-5f, 0.25f, nullptr, ws, need1,
                                     (float*)out, nullptr), UNS);
}

static void lambda_and_combine_cases() {
    void* p = dev(0);
    const float* f = (const float*)p;
    expect_reject(diffattn_lambda(f, f, f, f, 0, 64, 1, (float*)p, nullptr), INV);
    expect_reject(diffattn_lambda(f, f, f, f, 4, 64, 0, (float*)p, nullptr), INV);
    expect_reject(diffattn_lambda(f, f, f, (const float*)host(0), 4, 64, 1, (float*)p, nullptr), INV);
    CHECK(diffattn_lambda(f, f, f, f, 4, 64, 6, (float*)p, nullptr) == OK);
    CHECK(g_stub.H == 4 && g_stub.dim == 64 && g_stub.lambda_init == diffattn_lambda_init(6));
    CHECK(std::fabs(diffattn_lambda_init(1) - 0.2) < 1e-15);
    CHECK(std::isnan(diffattn_lambda_init(0)));
    expect_reject(diffattn_combine(f, f, f, 1, 2, 8, 96, 0, 0.f, 1.f, nullptr, (float*)p, nullptr), UNS);
    expect_reject(diffattn_combine(f, (const float*)dev(2), f, 1, 2, 8, 128, 0, 0.f, 1.f, nullptr,
                                   (float*)p, nullptr), INV);
    CHECK(diffattn_combine(f, f, f, 1, 2, 8, 128, 1, 1e-5f, 1.f, nullptr, (float*)p, nullptr) == OK);
    for (int s = 0; s <= 4; ++s) CHECK(std::strcmp(diffattn_status_string(s), "unknown status") != 0);
    CHECK(std::strcmp(diffattn_status_string(99), "unknown status") == 0);
    CHECK(std::strcmp(diffattn_status_string(-1), "unknown status") == 0);
}

// The error detail is thread-local: a failing call on another thread leaves
// this thread's message alone.
static void thread_local_error() {
    Prefill bad;
    bad.d = 48;
    CHECK(bad.call() == UNS);
    char mine[512];
    std::strncpy(mine, diffattn_last_error(), sizeof mine - 1);
    mine[sizeof mine - 1] = '\0';
    std::thread t([] {
        Prefill other;
        other.B = 0;
        CHECK(other.call() == INV);
        CHECK(std::strstr(diffattn_last_error(), "B=0") != nullptr);
    });
    t.join();
    CHECK(std::strcmp(mine, diffattn_last_error()) == 0);
    Prefill good;
    CHECK(good.call() == OK);
    CHECK(diffattn_last_error()[0] == '\0');
}

int main() {
    prefill_cases();
    prefill_v2_cases();
    decode_cases();
    lambda_and_combine_cases();
    thread_local_error();
    std::printf("abi host check: %d checks, %d failed\n", g_checks, g_fail);
    return g_fail ? 1 : 0;
}
