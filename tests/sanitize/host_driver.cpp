// Drives libkvq's C ABI on a fake device (HIP calls and kernel launches
// stubbed), for a build with the address and undefined-behaviour sanitizers:
// context creation for every mode and option, the table builders, and the
// host validation of every entry point.  Prints "host ok".
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kvq.h"
#include "stub_record.h"

#define CHECK(e)                                                                    \
    do {                                                                            \
        if (!(e)) {                                                                 \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #e, __LINE__);    \
            return 1;                                                               \
        }                                                                           \
    } while (0)

namespace {
// A fake device buffer: 256-byte aligned host memory (never dereferenced by
// the stubbed launches).
struct Buf {
    void *p;
    explicit Buf(size_t n) : p(std::aligned_alloc(256, (n + 255) / 256 * 256 + 256)) {}
    ~Buf() { std::free(p); }
    template <class T> T *as(size_t byte_off = 0) { return reinterpret_cast<T *>(static_cast<char *>(p) + byte_off); }
};

kvq_config base(int bits, int mode, int H)
{
    kvq_config c;
    std::memset(&c, 0, sizeof(c));
    c.d = 128;
    c.bits = bits;
    c.mode = mode;
    c.n_kv_heads = H;
    c.seed = 1234;
    return c;
}
}  // namespace

int main()
{
    // a release build of the host code: no bounds-check records
    CHECK(kvq_debug_build() == 0 && kvq_debug_take() == 0u);
    // tables without a context
    for (int b = 1; b <= 4; ++b) {
        float c[16], t[16];
        CHECK(kvq_codebook(b, c, t) == KVQ_OK);
        const int L = 1 << b;
        for (int j = 0; j < L; ++j) CHECK(c[j] == -c[L - 1 - j]);
        for (int j = 0; j + 1 < L; ++j) CHECK(c[j] < t[j] && t[j] < c[j + 1]);
    }
    float cc[16], tt[16];
    CHECK(kvq_codebook(0, cc, tt) == KVQ_E_INVAL && kvq_codebook(5, cc, tt) == KVQ_E_INVAL);
    CHECK(kvq_codebook(3, nullptr, tt) == KVQ_E_INVAL);
    CHECK(std::strlen(kvq_strerror((kvq_status)99)) > 0);

    const int H = 4;
    std::vector<float> S(128 * 128), Q(128 * 128, 0.f), Qbad(128 * 128, 0.f), cb(256 * 8);
    unsigned s = 7;
    auto rnd = [&]() { s = s * 1664525u + 1013904223u; return ((s >> 8) & 0xFFFF) / 65536.0f - 0.5f; };
    for (auto &v : S) v = rnd() * 4;
    for (auto &v : cb) v = rnd() * 3;
    for (int i = 0; i < 128; ++i) Q[i * 128 + i] = 1.f;
    Qbad = Q;
    Qbad[5] = 0.5f;
    std::vector<int8_t> sg(H * 128, 1), sgbad(H * 128, 1);
    sgbad[77] = 0;

    // creation: valid and invalid configurations
    kvq_ctx *ctx = nullptr;
    CHECK(kvq_create(nullptr, &ctx) == KVQ_E_INVAL);
    kvq_config c = base(3, KVQ_MODE_MSE, H);
    c.d = 64;
    CHECK(kvq_create(&c, &ctx) == KVQ_E_INVAL && ctx == nullptr);
    c = base(5, KVQ_MODE_MSE, H);
    CHECK(kvq_create(&c, &ctx) == KVQ_E_INVAL);
    c = base(3, KVQ_MODE_MSE, H);
    c.signs_k = sgbad.data();
    CHECK(kvq_create(&c, &ctx) == KVQ_E_INVAL);
    c = base(3, KVQ_MODE_MSE_QJL, H);
    CHECK(kvq_create(&c, &ctx) == KVQ_E_INVAL);  // no S
    c = base(3, KVQ_MODE_MSE, H);
    c.nsn_options = KVQ_NSN_ADAPTIVE_SCALE;  // an NSN option outside the NSN mode
    CHECK(kvq_create(&c, &ctx) == KVQ_E_INVAL);
    c = base(1, KVQ_MODE_NSN_VQ, H);
    c.vq_codebook = cb.data();
    c.nsn_options = 0x40;  // unknown option bit
    CHECK(kvq_create(&c, &ctx) == KVQ_E_INVAL);
    c.nsn_options = KVQ_NSN_ADAPTIVE_SCALE;
    CHECK(kvq_create(&c, &ctx) == KVQ_OK);
    CHECK(kvq_destroy(ctx) == KVQ_OK);
    c = base(3, KVQ_MODE_MSE, H);
    c.rotation = KVQ_ROTATION_DENSE;
    c.rot_Q = Qbad.data();
    CHECK(kvq_create(&c, &ctx) == KVQ_E_INVAL);  // not orthogonal
    c = base(3, KVQ_MODE_MSE_QJL, H);
    c.qjl_S = S.data();
    c.rotation = KVQ_ROTATION_DENSE;
    c.rot_Q = Q.data();
    kvq_ctx *dqjl = nullptr;
    kvq_status st = kvq_create(&c, &dqjl);
    CHECK(st == KVQ_OK);
    c = base(1, KVQ_MODE_NSN_VQ, H);
    c.vq_codebook = cb.data();
    c.rotation = KVQ_ROTATION_DENSE;
    c.rot_Q = Q.data();
    CHECK(kvq_create(&c, &ctx) == KVQ_E_UNSUPPORTED);

    std::vector<kvq_ctx *> all;
    for (int b = 1; b <= 4; ++b)
        for (int cbk = 0; cbk < 2; ++cbk) {
            c = base(b, KVQ_MODE_MSE, H);
            c.codebook = cbk;
            if (b == 2) c.signs_k = sg.data();
            CHECK(kvq_create(&c, &ctx) == KVQ_OK);
            all.push_back(ctx);
            float ct[16], tt2[16];
            std::vector<int8_t> sk(H * 128), sv(H * 128);
            CHECK(kvq_get_tables(ctx, ct, tt2, sk.data(), sv.data()) == KVQ_OK);
            for (int i = 0; i < H * 128; ++i) CHECK((sk[i] == 1 || sk[i] == -1) && (sv[i] == 1 || sv[i] == -1));
            CHECK(kvq_code_bytes_per_vec(ctx) == 16 * b);
        }
    kvq_ctx *mse = all[4];  // 3 bits, N(0,1) tables
    c = base(2, KVQ_MODE_MSE_QJL, H);
    c.qjl_S = S.data();
    kvq_ctx *qjl = nullptr;
    CHECK(kvq_create(&c, &qjl) == KVQ_OK);
    c = base(1, KVQ_MODE_NSN_VQ, H);
    c.vq_codebook = cb.data();
    kvq_ctx *nsn = nullptr;
    CHECK(kvq_create(&c, &nsn) == KVQ_OK);
    CHECK(kvq_get_tables(nsn, nullptr, nullptr, sg.data(), nullptr) == KVQ_E_INVAL);
    c = base(3, KVQ_MODE_MSE, H);
    c.rotation = KVQ_ROTATION_DENSE;
    c.rot_Q = Q.data();
    kvq_ctx *dense = nullptr;
    CHECK(kvq_create(&c, &dense) == KVQ_OK);

    // quantize
    const int64_t B = 2, T = 1000, Hq = 4 * H;
    Buf x(B * H * T * 256), codes(B * H * T * 64), norms(B * H * T * 4), q(B * 8 * H * 256), out(B * 8 * H * 512);
    Buf lg(B * 8 * H * T * 4), signs(B * H * T * 16), gamma(B * H * T * 4);
    void *st0 = nullptr;
    CHECK(kvq_quantize(mse, 2, x.p, B, H, T, codes.as<uint8_t>(), norms.as<float>(), nullptr, nullptr, st0) == KVQ_E_INVAL);
    CHECK(kvq_quantize(mse, 0, x.p, B, H + 1, T, codes.as<uint8_t>(), norms.as<float>(), nullptr, nullptr, st0) == KVQ_E_INVAL);
    CHECK(kvq_quantize(mse, 0, x.as<char>(2), B, H, T, codes.as<uint8_t>(), norms.as<float>(), nullptr, nullptr, st0) == KVQ_E_INVAL);
    const int calls0 = g_last.calls;
    CHECK(kvq_quantize(mse, 0, x.p, 0, H, T, codes.as<uint8_t>(), norms.as<float>(), nullptr, nullptr, st0) == KVQ_OK);
    CHECK(g_last.calls == calls0);  // empty call: nothing launched
    CHECK(kvq_quantize(mse, 1, x.p, B, H, T, codes.as<uint8_t>(), norms.as<float>(), nullptr, nullptr, st0) == KVQ_OK);
    CHECK(std::strcmp(g_last.what, "quantize") == 0 && g_last.a == 1 && g_last.c == T);
    CHECK(kvq_quantize(qjl, 0, x.p, B, H, T, codes.as<uint8_t>(), norms.as<float>(), nullptr, nullptr, st0) == KVQ_E_INVAL);
    CHECK(kvq_quantize(qjl, 0, x.p, B, H, T, codes.as<uint8_t>(), norms.as<float>(), signs.as<uint8_t>(), gamma.as<float>(), st0) == KVQ_OK);
    CHECK(kvq_quantize(qjl, 1, x.p, B, H, T, codes.as<uint8_t>(), norms.as<float>(), signs.as<uint8_t>(), gamma.as<float>(), st0) == KVQ_E_INVAL);
    CHECK(kvq_quantize(dense, 0, x.p, B, H, T, codes.as<uint8_t>(), norms.as<float>(), nullptr, nullptr, st0) == KVQ_OK);
    CHECK(std::strcmp(g_last.what, "quantize_dense") == 0 && g_last.a == B * H * T);
    CHECK(kvq_quantize(dqjl, 0, x.p, B, H, T, codes.as<uint8_t>(), norms.as<float>(), signs.as<uint8_t>(), gamma.as<float>(), st0) == KVQ_OK);
    CHECK(std::strcmp(g_last.what, "quantize_dense_qjl") == 0 && g_last.a == B * H * T);
    CHECK(kvq_quantize(dqjl, 1, x.p, B, H, T, codes.as<uint8_t>(), norms.as<float>(), nullptr, nullptr, st0) == KVQ_OK);
    CHECK(std::strcmp(g_last.what, "quantize_dense") == 0);
    CHECK(kvq_quantize_kv(mse, x.p, x.p, B, H, T, codes.as<uint8_t>(), norms.as<float>(), codes.as<uint8_t>(), norms.as<float>(), st0) == KVQ_OK);
    CHECK(kvq_quantize_kv(qjl, x.p, x.p, B, H, T, codes.as<uint8_t>(), norms.as<float>(), codes.as<uint8_t>(), norms.as<float>(), st0) == KVQ_E_INVAL);

    // logits: group sizes 1, 2, 4, 8 are built; 3 is not; 6 heads do not divide
    for (int G : {1, 2, 4, 8})
        CHECK(kvq_logits(mse, q.p, B, H * G, T, codes.as<uint8_t>(), norms.as<float>(), nullptr, nullptr, lg.as<float>(), st0) == KVQ_OK);
    CHECK(kvq_logits(mse, q.p, B, H * 3, T, codes.as<uint8_t>(), norms.as<float>(), nullptr, nullptr, lg.as<float>(), st0) == KVQ_E_UNSUPPORTED);
    CHECK(kvq_logits(mse, q.p, B, 6, T, codes.as<uint8_t>(), norms.as<float>(), nullptr, nullptr, lg.as<float>(), st0) == KVQ_E_INVAL);
    CHECK(kvq_logits(qjl, q.p, B, Hq, T, codes.as<uint8_t>(), norms.as<float>(), nullptr, nullptr, lg.as<float>(), st0) == KVQ_E_INVAL);
    CHECK(kvq_logits(qjl, q.p, B, Hq, T, codes.as<uint8_t>(), norms.as<float>(), signs.as<uint8_t>(), gamma.as<float>(), lg.as<float>(), st0) == KVQ_OK);

    // decode: workspace sizes, split clamping, group sizes
    const size_t wsb = kvq_attn_decode_ws_bytes(mse, B, Hq, T);
    CHECK(wsb > 0 && kvq_attn_decode_ws_bytes(nullptr, B, Hq, T) == 0);
    Buf ws(wsb);
    CHECK(kvq_attn_decode(mse, q.p, B, Hq, T, codes.as<uint8_t>(), norms.as<float>(), codes.as<uint8_t>(), norms.as<float>(), 0.f, out.as<float>(), ws.p, wsb - 1, st0) == KVQ_E_WORKSPACE);
    CHECK(kvq_attn_decode(mse, q.p, B, Hq, T, codes.as<uint8_t>(), norms.as<float>(), codes.as<uint8_t>(), norms.as<float>(), 0.f, out.as<float>(), ws.as<char>(16), wsb, st0) == KVQ_E_INVAL);
    CHECK(kvq_attn_decode(mse, q.p, B, Hq, T, codes.as<uint8_t>(), norms.as<float>(), codes.as<uint8_t>(), norms.as<float>(), -1.f, out.as<float>(), ws.p, wsb, st0) == KVQ_E_INVAL);
    CHECK(kvq_attn_decode(mse, q.p, B, Hq, T, codes.as<uint8_t>(), norms.as<float>(), codes.as<uint8_t>(), norms.as<float>(), 0.f, out.as<float>(), ws.p, wsb, st0) == KVQ_OK);
    CHECK(std::strcmp(g_last.what, "decode") == 0 && g_last.n_split >= 1 && g_last.n_split <= (T + 63) / 64);
    if (const char *e = std::getenv("KVQ_SPLITS")) {  // the automatic count replaced (then clamped)
        const int want = std::atoi(e);
        CHECK(want > 0 && g_last.n_split == (want < (T + 63) / 64 ? want : (T + 63) / 64));
    }
    CHECK(kvq_attn_decode_splits(mse, q.p, B, Hq, T, codes.as<uint8_t>(), norms.as<float>(), codes.as<uint8_t>(), norms.as<float>(), 0.f, out.as<float>(), ws.p, wsb, 1000000, st0) == KVQ_OK);
    CHECK(g_last.n_split == (T + 63) / 64);
    CHECK(kvq_attn_decode(mse, q.p, B, H * 8, T, codes.as<uint8_t>(), norms.as<float>(), codes.as<uint8_t>(), norms.as<float>(), 0.f, out.as<float>(), ws.p, wsb, st0) == KVQ_E_UNSUPPORTED);
    CHECK(kvq_attn_decode(mse, q.p, B, Hq, 0, codes.as<uint8_t>(), norms.as<float>(), codes.as<uint8_t>(), norms.as<float>(), 0.f, out.as<float>(), ws.p, wsb, st0) == KVQ_E_INVAL);
    CHECK(kvq_attn_decode(qjl, q.p, B, Hq, T, codes.as<uint8_t>(), norms.as<float>(), codes.as<uint8_t>(), norms.as<float>(), 0.f, out.as<float>(), ws.p, wsb, st0) == KVQ_E_INVAL);

    // no-allocation decode: split count lowered to fit the fixed scratch, then rejected
    CHECK(kvq_attn_decode_noalloc(mse, q.p, B, Hq, T, codes.as<uint8_t>(), norms.as<float>(), codes.as<uint8_t>(), norms.as<float>(), 0.f, out.as<float>(), st0) == KVQ_OK);
    CHECK(std::strcmp(g_last.what, "decode_noalloc") == 0 && g_last.n_split >= 1);
    {
        const int64_t Bb = 900;  // 900 x 16 query heads at one split: 7.5 MB of partials, fits
        Buf qb(Bb * Hq * 256), ob(Bb * Hq * 512);
        st = kvq_attn_decode_noalloc(mse, qb.p, Bb, Hq, 100000, codes.as<uint8_t>(), norms.as<float>(), codes.as<uint8_t>(), norms.as<float>(), 0.f, ob.as<float>(), st0);
        CHECK(st == KVQ_OK);
        const size_t need = 65536 + (size_t)Bb * Hq * g_last.n_split * 520;
        CHECK(need <= KVQ_NOALLOC_SCRATCH_BYTES);
        CHECK(g_last.n_split >= 1);
    }
    {
        const int64_t Bb = 1100;  // 17600 query heads: not even one split fits
        Buf qb(Bb * Hq * 256), ob(Bb * Hq * 512);
        CHECK(kvq_attn_decode_noalloc(mse, qb.p, Bb, Hq, 10, codes.as<uint8_t>(), norms.as<float>(), codes.as<uint8_t>(), norms.as<float>(), 0.f, ob.as<float>(), st0) == KVQ_E_WORKSPACE);
    }

    // streaming cache
    const int64_t Tcap = T + 100, R = 40, Rcap = 64;
    const size_t sws = kvq_attn_decode_stream_ws_bytes(mse, B, Hq, Tcap);
    Buf sw(sws), tail(B * H * Rcap * 256);
    CHECK(kvq_attn_decode_stream(mse, q.p, B, Hq, T, Tcap, codes.as<uint8_t>(), norms.as<float>(), codes.as<uint8_t>(), norms.as<float>(), R, Rcap, tail.p, tail.p, 0.f, out.as<float>(), sw.p, sws, st0) == KVQ_OK);
    CHECK(kvq_attn_decode_stream(mse, q.p, B, Hq, Tcap + 1, Tcap, codes.as<uint8_t>(), norms.as<float>(), codes.as<uint8_t>(), norms.as<float>(), R, Rcap, tail.p, tail.p, 0.f, out.as<float>(), sw.p, sws, st0) == KVQ_E_INVAL);
    CHECK(kvq_attn_decode_stream(mse, q.p, B, Hq, 0, Tcap, nullptr, nullptr, nullptr, nullptr, 0, Rcap, tail.p, tail.p, 0.f, out.as<float>(), sw.p, sws, st0) == KVQ_E_INVAL);
    CHECK(kvq_attn_decode_stream(dense, q.p, B, Hq, T, Tcap, codes.as<uint8_t>(), norms.as<float>(), codes.as<uint8_t>(), norms.as<float>(), R, Rcap, tail.p, tail.p, 0.f, out.as<float>(), sw.p, sws, st0) == KVQ_E_UNSUPPORTED);
    CHECK(kvq_flush(mse, tail.p, tail.p, B, H, R, Rcap, codes.as<uint8_t>(), norms.as<float>(), codes.as<uint8_t>(), norms.as<float>(), T, Tcap, st0) == KVQ_OK);
    CHECK(kvq_flush(mse, tail.p, tail.p, B, H, R, Rcap, codes.as<uint8_t>(), norms.as<float>(), codes.as<uint8_t>(), norms.as<float>(), Tcap - R + 1, Tcap, st0) == KVQ_E_INVAL);

    // NSN-VQ
    const size_t nws = kvq_nsn_vq_ws_bytes(nsn, H, T);
    Buf nw(nws), o(H * 512), s1(H * T * 4);
    CHECK(kvq_nsn_vq_quantize(nsn, x.p, H, T, codes.as<uint8_t>(), s1.as<float>(), s1.as<float>(), o.as<float>(), nw.p, nws - 4, st0) == KVQ_E_WORKSPACE);
    CHECK(kvq_nsn_vq_quantize(nsn, x.p, H, T, codes.as<uint8_t>(), s1.as<float>(), s1.as<float>(), o.as<float>(), nw.p, nws, st0) == KVQ_OK);
    CHECK(kvq_nsn_vq_quantize(mse, x.p, H, T, codes.as<uint8_t>(), s1.as<float>(), s1.as<float>(), o.as<float>(), nw.p, nws, st0) == KVQ_E_INVAL);
    CHECK(kvq_nsn_logits(nsn, q.p, 1, H * 3, T, codes.as<uint8_t>(), s1.as<float>(), s1.as<float>(), o.as<float>(), lg.as<float>(), st0) == KVQ_E_INVAL);
    CHECK(kvq_nsn_logits(nsn, q.p, 1, H * 8, T, codes.as<uint8_t>(), s1.as<float>(), s1.as<float>(), o.as<float>(), lg.as<float>(), st0) == KVQ_OK);
    const size_t ndw = kvq_nsn_attn_decode_ws_bytes(nsn, 1, Hq, T);
    Buf nd(ndw);
    CHECK(kvq_nsn_attn_decode(nsn, q.p, 1, Hq, T, codes.as<uint8_t>(), s1.as<float>(), s1.as<float>(), o.as<float>(), codes.as<uint8_t>(), s1.as<float>(), s1.as<float>(), o.as<float>(), 0.f, out.as<float>(), nd.p, ndw, st0) == KVQ_OK);
    CHECK(g_last.n_split >= 1 && g_last.n_split <= (T + 63) / 64);
    CHECK(kvq_nsn_attn_decode(nsn, q.p, 1, Hq, T, codes.as<uint8_t>(), s1.as<float>(), s1.as<float>(), o.as<float>(), codes.as<uint8_t>(), s1.as<float>(), s1.as<float>(), o.as<float>(), 0.f, out.as<float>(), nd.p, ndw - 1, st0) == KVQ_E_WORKSPACE);

    // NSN-VQ with double-quantised byproducts
    {
        const size_t qws = kvq_nsn_vq_dq_ws_bytes(nsn, H, T);
        CHECK(qws > kvq_nsn_vq_ws_bytes(nsn, H, T));
        Buf qw(qws), s1q(H * T), s1p(H * T * 8), s2(H * T * 4), oq(H * 64), op(H * 8);
        CHECK(kvq_nsn_vq_quantize_dq(nsn, x.p, H, T, codes.as<uint8_t>(), s1q.as<uint8_t>(), s1p.as<float>(), s2.as<float>(), oq.as<uint8_t>(), op.as<float>(), qw.p, qws, st0) == KVQ_OK);
        CHECK(std::strcmp(g_last.what, "nsn_vq_dq") == 0 && g_last.a == H && g_last.b == T);
        CHECK(kvq_nsn_vq_quantize_dq(nsn, x.p, H, T, codes.as<uint8_t>(), s1q.as<uint8_t>(), s1p.as<float>(), s2.as<float>(), oq.as<uint8_t>(), op.as<float>(), qw.p, qws - 1, st0) == KVQ_E_WORKSPACE);
        CHECK(kvq_nsn_vq_quantize_dq(nsn, x.p, H, T, codes.as<uint8_t>(), s1q.as<uint8_t>(), s1p.as<float>(4), s2.as<float>(), oq.as<uint8_t>(), op.as<float>(), qw.p, qws, st0) == KVQ_E_INVAL);
        CHECK(kvq_nsn_vq_quantize_dq(mse, x.p, H, T, codes.as<uint8_t>(), s1q.as<uint8_t>(), s1p.as<float>(), s2.as<float>(), oq.as<uint8_t>(), op.as<float>(), qw.p, qws, st0) == KVQ_E_INVAL);
        CHECK(kvq_nsn_logits_dq(nsn, q.p, 1, H * 8, T, codes.as<uint8_t>(), s1q.as<uint8_t>(), s1p.as<float>(), s2.as<float>(), oq.as<uint8_t>(), op.as<float>(), lg.as<float>(), st0) == KVQ_OK);
        CHECK(std::strcmp(g_last.what, "nsn_logits_dq") == 0);
        CHECK(kvq_nsn_logits_dq(nsn, q.p, 1, H * 8, T, codes.as<uint8_t>(), nullptr, s1p.as<float>(), s2.as<float>(), oq.as<uint8_t>(), op.as<float>(), lg.as<float>(), st0) == KVQ_E_INVAL);
        const size_t ddw = kvq_nsn_attn_decode_ws_bytes(nsn, 1, Hq, T);
        Buf dd(ddw);
        CHECK(kvq_nsn_attn_decode_dq(nsn, q.p, 1, Hq, T, codes.as<uint8_t>(), s1q.as<uint8_t>(), s1p.as<float>(), s2.as<float>(), oq.as<uint8_t>(), op.as<float>(), codes.as<uint8_t>(), s1q.as<uint8_t>(), s1p.as<float>(), s2.as<float>(), oq.as<uint8_t>(), op.as<float>(), 0.f, out.as<float>(), dd.p, ddw, 0, st0) == KVQ_OK);
        CHECK(std::strcmp(g_last.what, "nsn_decode_dq") == 0 && g_last.n_split >= 1);
        CHECK(kvq_nsn_attn_decode_dq(nsn, q.p, 1, Hq, T, codes.as<uint8_t>(), s1q.as<uint8_t>(), s1p.as<float>(), s2.as<float>(), oq.as<uint8_t>(), op.as<float>(), codes.as<uint8_t>(), s1q.as<uint8_t>(), s1p.as<float>(), s2.as<float>(), oq.as<uint8_t>(), nullptr, 0.f, out.as<float>(), dd.p, ddw, 0, st0) == KVQ_E_INVAL);
        CHECK(kvq_nsn_attn_decode_dq(nsn, q.p, 1, Hq, T, codes.as<uint8_t>(), s1q.as<uint8_t>(), s1p.as<float>(), s2.as<float>(), oq.as<uint8_t>(), op.as<float>(), codes.as<uint8_t>(), s1q.as<uint8_t>(), s1p.as<float>(), s2.as<float>(), oq.as<uint8_t>(), op.as<float>(), 0.f, out.as<float>(), dd.p, ddw - 1, 0, st0) == KVQ_E_WORKSPACE);
    }
    {
        // the codebook option: accepted in the NSN mode only
        kvq_config cd = base(1, KVQ_MODE_NSN_VQ, H);
        cd.vq_codebook = cb.data();
        cd.nsn_options = KVQ_NSN_DQ_CODEBOOK | KVQ_NSN_ADAPTIVE_SCALE;
        kvq_ctx *cx = nullptr;
        CHECK(kvq_create(&cd, &cx) == KVQ_OK && kvq_destroy(cx) == KVQ_OK);
        cd = base(3, KVQ_MODE_MSE, H);
        cd.nsn_options = KVQ_NSN_DQ_CODEBOOK;
        CHECK(kvq_create(&cd, &cx) == KVQ_E_INVAL);
    }

    // gain-shape residual quantisation
    {
        std::vector<float> gt(2 * (256 * 32 + 16));
        for (auto &v : gt) v = rnd();
        for (int st = 0; st < 2; ++st)
            for (int l = 0; l < 16; ++l) gt[st * (256 * 32 + 16) + 256 * 32 + l] = 0.5f + 0.25f * l;
        kvq_config cg = base(1, KVQ_MODE_GSRQ, H);
        kvq_ctx *gq = nullptr;
        CHECK(kvq_create(&cg, &gq) == KVQ_E_INVAL);  // no tables
        cg.gsrq_tables = gt.data();
        gt[256 * 32 + 5] = gt[256 * 32 + 4];  // levels not increasing
        CHECK(kvq_create(&cg, &gq) == KVQ_E_INVAL);
        gt[256 * 32 + 5] = 0.5f + 0.25f * 5;
        cg.rotation = KVQ_ROTATION_DENSE;
        cg.rot_Q = Q.data();
        CHECK(kvq_create(&cg, &gq) == KVQ_E_UNSUPPORTED);
        cg.rotation = KVQ_ROTATION_HADAMARD;
        cg.rot_Q = nullptr;
        CHECK(kvq_create(&cg, &gq) == KVQ_OK);
        CHECK(kvq_code_bytes_per_vec(gq) == 12);
        const size_t gws = kvq_gsrq_ws_bytes(gq, H, T);
        Buf gw(gws), gc(H * T * 12), gs1(H * T * 4), go(H * 512);
        CHECK(kvq_gsrq_quantize(gq, x.p, H, T, gc.as<uint8_t>(), gs1.as<float>(), gs1.as<float>(), go.as<float>(), gw.p, gws, st0) == KVQ_OK);
        CHECK(std::strcmp(g_last.what, "gsrq") == 0 && g_last.a == H && g_last.b == T);
        CHECK(kvq_gsrq_quantize(gq, x.p, H, T, gc.as<uint8_t>(), gs1.as<float>(), gs1.as<float>(), go.as<float>(), gw.p, gws - 1, st0) == KVQ_E_WORKSPACE);
        CHECK(kvq_gsrq_quantize(nsn, x.p, H, T, gc.as<uint8_t>(), gs1.as<float>(), gs1.as<float>(), go.as<float>(), gw.p, gws, st0) == KVQ_E_INVAL);
        CHECK(kvq_quantize(gq, 0, x.p, 1, H, T, codes.as<uint8_t>(), norms.as<float>(), nullptr, nullptr, st0) == KVQ_E_INVAL);
        CHECK(kvq_gsrq_logits(gq, q.p, 1, H * 8, T, gc.as<uint8_t>(), gs1.as<float>(), gs1.as<float>(), go.as<float>(), lg.as<float>(), st0) == KVQ_OK);
        CHECK(kvq_gsrq_logits(gq, q.p, 1, H * 3, T, gc.as<uint8_t>(), gs1.as<float>(), gs1.as<float>(), go.as<float>(), lg.as<float>(), st0) == KVQ_E_INVAL);
        const size_t gdw = kvq_nsn_attn_decode_ws_bytes(gq, 1, Hq, T);
        Buf gd(gdw);
        CHECK(kvq_gsrq_attn_decode(gq, q.p, 1, Hq, T, gc.as<uint8_t>(), gs1.as<float>(), gs1.as<float>(), go.as<float>(), gc.as<uint8_t>(), gs1.as<float>(), gs1.as<float>(), go.as<float>(), 0.f, out.as<float>(), gd.p, gdw, 0, st0) == KVQ_OK);
        CHECK(std::strcmp(g_last.what, "gsrq_decode") == 0 && g_last.n_split >= 1);
        CHECK(kvq_gsrq_attn_decode(gq, q.p, 1, H * 8, T, gc.as<uint8_t>(), gs1.as<float>(), gs1.as<float>(), go.as<float>(), gc.as<uint8_t>(), gs1.as<float>(), gs1.as<float>(), go.as<float>(), 0.f, out.as<float>(), gd.p, gdw, 0, st0) == KVQ_E_INVAL);
        CHECK(kvq_gsrq_attn_decode(gq, q.p, 1, Hq, T, gc.as<uint8_t>(), gs1.as<float>(), gs1.as<float>(), go.as<float>(), gc.as<uint8_t>(), gs1.as<float>(), gs1.as<float>(), go.as<float>(), 0.f, out.as<float>(), gd.p, gdw - 1, 0, st0) == KVQ_E_WORKSPACE);
        CHECK(kvq_destroy(gq) == KVQ_OK);
    }

    // NSN-VQ streaming cache: flush groups of Gs tokens, decode over packed + window
    {
        const int64_t Gs = 128, Tc = 1024, Rc = 192, Tn = 512, Rn = 40;
        Buf pc(B * H * Tc * 16), ps(B * H * Tc * 4), po(B * H * (Tc / Gs) * 512), win(B * H * Rc * 256);
        const size_t fws = kvq_nsn_flush_ws_bytes(nsn, B, Gs);
        CHECK(fws > 0 && kvq_nsn_flush_ws_bytes(nullptr, B, Gs) == 0);
        Buf fw(fws);
        auto flush = [&](kvq_ctx *cx, int64_t g, int64_t t0, int64_t tcap, size_t wsb) {
            return kvq_nsn_flush(cx, win.p, win.p, B, H, g, Rc, pc.as<uint8_t>(), ps.as<float>(), ps.as<float>(),
                                 po.as<float>(), pc.as<uint8_t>(), ps.as<float>(), ps.as<float>(), po.as<float>(), t0,
                                 tcap, fw.p, wsb, st0);
        };
        CHECK(flush(nsn, Gs, 256, Tc, fws) == KVQ_OK);
        CHECK(std::strcmp(g_last.what, "nsn_vq_strided") == 0 && g_last.a == B * H && g_last.b == Gs && g_last.c == Tc);
        CHECK(flush(nsn, Gs, 100, Tc, fws) == KVQ_E_INVAL);       // T0 not a multiple of Gs
        CHECK(flush(nsn, 96, 192, Tc, fws) == KVQ_E_INVAL);       // Gs not a multiple of 64
        CHECK(flush(nsn, Gs, Tc, Tc, fws) == KVQ_E_INVAL);        // past the capacity
        CHECK(flush(nsn, 256, 0, 1024, fws) == KVQ_E_INVAL);      // Gs > R_cap
        CHECK(flush(nsn, Gs, 0, 1000, fws) == KVQ_E_INVAL);       // T_cap not a multiple of Gs
        CHECK(flush(mse, Gs, 0, Tc, fws) == KVQ_E_INVAL);         // not an NSN context
        CHECK(flush(nsn, Gs, 0, Tc, fws - 1) == KVQ_E_WORKSPACE);
        const size_t dws = kvq_nsn_attn_decode_stream_ws_bytes(nsn, B, Hq, Tc);
        CHECK(dws > 0);
        Buf dw(dws);
        auto dec = [&](int64_t hq, int64_t t, int64_t r, bool packed, size_t wsb, int32_t ns) {
            return kvq_nsn_attn_decode_stream(
                nsn, q.p, B, hq, t, Tc, Gs, packed ? pc.as<uint8_t>() : nullptr, packed ? ps.as<float>() : nullptr,
                packed ? ps.as<float>() : nullptr, packed ? po.as<float>() : nullptr, packed ? pc.as<uint8_t>() : nullptr,
                packed ? ps.as<float>() : nullptr, packed ? ps.as<float>() : nullptr, packed ? po.as<float>() : nullptr,
                r, Rc, win.p, win.p, 0.f, out.as<float>(), dw.p, wsb, ns, st0);
        };
        CHECK(dec(Hq, Tn, Rn, true, dws, 0) == KVQ_OK);
        CHECK(std::strcmp(g_last.what, "nsn_decode_stream") == 0 && g_last.n_split >= 1 && g_last.n_split <= Tn / 64);
        CHECK(dec(Hq, Tn, Rn, true, dws, 1000) == KVQ_OK && g_last.n_split == Tn / 64);
        CHECK(dec(Hq, 500, Rn, true, dws, 0) == KVQ_E_INVAL);     // T not a multiple of Gs
        CHECK(dec(H * 8, Tn, Rn, true, dws, 0) == KVQ_E_INVAL);   // 8 query heads per KV head
        CHECK(dec(Hq, 0, 0, true, dws, 0) == KVQ_E_INVAL);        // nothing to attend to
        CHECK(dec(Hq, 0, Rn, false, dws, 0) == KVQ_OK);           // window only
        CHECK(dec(Hq, Tn, 0, true, dws, 0) == KVQ_OK);            // packed only
        CHECK(dec(Hq, Tn, Rn, false, dws, 0) == KVQ_E_INVAL);     // packed tokens without arrays
        CHECK(dec(Hq, Tn, Rn, true, dws - 1, 0) == KVQ_E_WORKSPACE);
        CHECK(dec(Hq, Tc + Gs, Rn, true, dws, 0) == KVQ_E_INVAL); // T > T_cap
    }

    for (kvq_ctx *p : all) CHECK(kvq_destroy(p) == KVQ_OK);
    CHECK(kvq_destroy(qjl) == KVQ_OK && kvq_destroy(nsn) == KVQ_OK && kvq_destroy(dense) == KVQ_OK);
    CHECK(kvq_destroy(dqjl) == KVQ_OK);
    CHECK(kvq_destroy(nullptr) == KVQ_OK);
    std::printf("host ok\n");
    return 0;
}
