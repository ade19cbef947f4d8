// Drives the library's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
// against the host-only runtime stand-in (sim_runtime.cpp): no kernel runs.
//
//   host_check FOLD_FILE
//
// 1. Each line of FOLD_FILE holds the 256 bins of a quantize exponent histogram (decimal
//    integers); one line of output per input, the exactly rounded sum as a hex float.
// 2. Every entry point is called with valid arguments at shapes that reach each of its
//    launch paths, on buffers allocated with their exact sizes (workspaces of exactly the
//    size that the library asks for): each call must return QLORA_OK and launch kernels
//    within the hardware's limits.
// 3. Error cases (null, misaligned and undersized arguments, shapes out of range): each call
//    must return its documented status and launch nothing.
// The last line of output is "OK <checks>"; the first failed check prints "FAIL ..." and
// the program exits with status 1.  Sanitizer reports end the program with their own status.
#include <cinttypes>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <sstream>
#include <string>
#include <utility>
#include <vector>

#include "qlora.h"
#include "qlora_host.h"
#include "sim_runtime.h"

namespace {

int g_checks = 0;

#define CHECK(cond, ...)                                      \
  do {                                                        \
    ++g_checks;                                               \
    if (!(cond)) {                                            \
      std::printf("FAIL line %d: %s: ", __LINE__, #cond);     \
      std::printf(__VA_ARGS__);                               \
      std::printf("\n");                                      \
      std::exit(1);                                           \
    }                                                         \
  } while (0)

// An exact-size, 256-byte-aligned host buffer standing in for device memory.
struct Buf {
  void* p = nullptr;
  size_t n = 0;
  Buf() = default;
  explicit Buf(size_t bytes) : n(bytes) {
    if (posix_memalign(&p, 256, bytes ? bytes : 1) != 0) std::abort();
    std::memset(p, 0, bytes ? bytes : 1);
  }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
  Buf(Buf&& o) noexcept : p(o.p), n(o.n) { o.p = nullptr; }
  Buf& operator=(Buf&& o) noexcept {
    std::swap(p, o.p);
    std::swap(n, o.n);
    return *this;
  }
  ~Buf() { std::free(p); }
  template <class T>
  T* as() const { return static_cast<T*>(p); }
};

// The buffers of one quantized [d_out, d_in] weight.
struct Weight {
  Buf codes, code8, c2s, mu;
  qlora_nf4dq_t q{};
  Weight(int64_t d_out, int64_t d_in, int codebook = QLORA_CB_NF4, int dq = QLORA_DQ_E4M3) {
    size_t cb = 0, c8 = 0, cs = 0;
    const int st = qlora_format_sizes(d_out, d_in, dq, &cb, &c8, &cs);
    CHECK(st == QLORA_OK, "format_sizes %" PRId64 "x%" PRId64 " -> %d", d_out, d_in, st);
    codes = Buf(cb);
    code8 = Buf(c8);
    if (cs) c2s = Buf(cs);
    if (dq != QLORA_DQ_NONE) mu = Buf(4);
    q.codes = codes.as<uint8_t>();
    q.code8 = code8.as<uint8_t>();
    q.c2s = c2s.as<float>();
    q.mu = mu.as<float>();
    q.d_out = d_out;
    q.d_in = d_in;
    q.block1 = 64;
    q.block2 = 256;
    q.codebook = codebook;
    q.dq_format = dq;
  }
};

size_t bf16(int64_t a, int64_t b) { return (size_t)(a * b * 2); }

size_t ws_need(int op, int64_t M, const qlora_nf4dq_t& q, int32_t r) {
  size_t n = 0;
  const int st = qlora_workspace_size_fmt(op, M, q.d_out, q.d_in, r, q.dq_format, &n);
  CHECK(st == QLORA_OK, "workspace_size op %d M %" PRId64 " -> %d", op, M, st);
  CHECK(n >= QLORA_WS_COUNTER_BYTES && n % 256 == 0, "workspace %zu bytes", n);
  return n;
}

// Runs `call`, which must return `want`; a success must launch kernels within limits, an
// error must launch nothing.
template <class F>
void expect(const char* what, int want, F call) {
  const size_t before = sim::launches();
  const int bad = sim::bad_launches();
  const int st = call();
  CHECK(st == want, "%s: status %d, want %d", what, st, want);
  if (want == QLORA_OK) {
    CHECK(sim::launches() > before, "%s: no kernel launched", what);
    CHECK(sim::bad_launches() == bad, "%s: a launch outside the hardware's limits", what);
  } else {
    CHECK(sim::launches() == before, "%s: failed with status %d after launching kernels", what, st);
  }
}

void fold(const char* path) {
  std::ifstream in(path);
  CHECK(in.good(), "cannot open %s", path);
  std::string line;
  while (std::getline(in, line)) {
    if (line.empty()) continue;
    std::istringstream ss(line);
    unsigned long long hist[256];
    for (int e = 0; e < 256; ++e) CHECK(static_cast<bool>(ss >> hist[e]), "short histogram line");
    std::printf("FOLD %a\n", qlora::exact_sum_to_double(hist));
  }
}

void sizes() {
  const int64_t shapes[][2] = {{16, 64}, {272, 320}, {4096, 4096}, {28672, 8192}, {1 << 22, 1024}, {1024, 1 << 22}};
  for (auto& s : shapes)
    for (int dq = QLORA_DQ_E4M3; dq <= QLORA_DQ_NONE; ++dq) {
      size_t a = 0, b = 0, c = 0;
      CHECK(qlora_format_sizes(s[0], s[1], dq, &a, &b, &c) == QLORA_OK, "sizes");
      const int64_t n = s[0] * s[1], nb = n / 64;
      CHECK(a == (size_t)(n / 2), "codes bytes");
      CHECK(b == (size_t)(dq == QLORA_DQ_NONE ? 4 * nb : nb), "code8 bytes");
      CHECK(c == (dq == QLORA_DQ_NONE ? 0 : (size_t)(4 * ((nb + 255) / 256))), "c2s bytes %zu", c);
      for (int op = QLORA_OP_QUANTIZE; op <= QLORA_OP_BWD; ++op)
        for (int64_t M : {int64_t(1), int64_t(16), int64_t(17), int64_t(1023), int64_t(1024), int64_t(1) << 20,
                          (int64_t(1) << 24) - 1}) {
          size_t w = 0;
          CHECK(qlora_workspace_size_fmt(op, M, s[0], s[1], 64, dq, &w) == QLORA_OK, "ws size");
          CHECK(w >= QLORA_WS_COUNTER_BYTES, "ws head");
        }
    }
  size_t w = 0;
  expect("ws M = 2^24", QLORA_ERR_INVALID_ARG, [&] { return qlora_workspace_size(QLORA_OP_FWD, 1 << 24, 64, 64, 8, &w); });
  expect("ws r = 129", QLORA_ERR_INVALID_ARG, [&] { return qlora_workspace_size(QLORA_OP_FWD, 1, 64, 64, 129, &w); });
  expect("ws d_in % 64", QLORA_ERR_BAD_SHAPE, [&] { return qlora_workspace_size(QLORA_OP_FWD, 1, 64, 96, 8, &w); });
  expect("ws d_out > 2^22", QLORA_ERR_BAD_SHAPE,
         [&] { return qlora_workspace_size(QLORA_OP_FWD, 1, (1 << 22) + 16, 64, 8, &w); });
  expect("ws d_out d_in > 2^32", QLORA_ERR_BAD_SHAPE,
         [&] { return qlora_workspace_size(QLORA_OP_FWD, 1, 1 << 22, 2048, 8, &w); });
  float cb[16];
  for (int c = QLORA_CB_NF4; c <= QLORA_CB_FP4; ++c) CHECK(qlora_codebook(c, cb) == QLORA_OK, "codebook %d", c);
  CHECK(qlora_codebook(3, cb) == QLORA_ERR_INVALID_ARG, "codebook 3");
  for (int s = 1; s >= -8; --s) CHECK(qlora_strerror(s) && std::strlen(qlora_strerror(s)) > 0, "strerror %d", s);
}

void quantize_paths() {
  const int64_t shapes[][2] = {{272, 320}, {1024, 4096}};
  for (auto& s : shapes)
    for (int cb = QLORA_CB_NF4; cb <= QLORA_CB_FP4; ++cb)
      for (int dq = QLORA_DQ_E4M3; dq <= QLORA_DQ_NONE; ++dq) {
        Weight w(s[0], s[1], cb, dq);
        Buf W(4 * s[0] * s[1]), Wb(bf16(s[0], s[1])), out(bf16(s[0], s[1]));
        const size_t need = ws_need(QLORA_OP_QUANTIZE, 1, w.q, 1);
        Buf ws(need);
        float mu = -1.f;
        expect("quantize", QLORA_OK, [&] { return qlora_quantize(W.as<float>(), &w.q, &mu, ws.p, need, nullptr); });
        expect("quantize bf16", QLORA_OK,
               [&] { return qlora_quantize_bf16(Wb.as<uint16_t>(), &w.q, &mu, ws.p, need, nullptr); });
        expect("quantize small ws", QLORA_ERR_WORKSPACE,
               [&] { return qlora_quantize(W.as<float>(), &w.q, &mu, ws.p, need - 1, nullptr); });
        expect("dequantize", QLORA_OK, [&] { return qlora_dequantize(&w.q, out.as<uint16_t>(), nullptr); });
        Buf A(bf16(16, s[1])), B(bf16(s[0], 16));
        expect("merge", QLORA_OK, [&] {
          return qlora_merge(&w.q, A.as<uint16_t>(), B.as<uint16_t>(), 16, 32.f, out.as<uint16_t>(), nullptr);
        });
      }
  Weight w(272, 320);
  Buf W(4 * 272 * 320 + 4);
  const size_t need = ws_need(QLORA_OP_QUANTIZE, 1, w.q, 1);
  Buf ws(need);
  expect("quantize misaligned W", QLORA_ERR_INVALID_ARG,
         [&] { return qlora_quantize(reinterpret_cast<const float*>(W.as<char>() + 4), &w.q, nullptr, ws.p, need, nullptr); });
  expect("quantize null ws", QLORA_ERR_WORKSPACE, [&] { return qlora_quantize(W.as<float>(), &w.q, nullptr, nullptr, need, nullptr); });
  qlora_nf4dq_t bad = w.q;
  bad.block1 = 32;
  expect("quantize block 32", QLORA_ERR_UNSUPPORTED, [&] { return qlora_quantize(W.as<float>(), &bad, nullptr, ws.p, need, nullptr); });
  bad = w.q;
  bad.code8 = nullptr;
  expect("dequantize null code8", QLORA_ERR_INVALID_ARG, [&] { return qlora_dequantize(&bad, W.as<uint16_t>(), nullptr); });
}

// One linear layer's activations, adapters and outputs at M tokens.
struct Layer {
  Buf X, A, B, Y, T, dY, dX, dA, dB;
  Layer(const qlora_nf4dq_t& q, int64_t M, int32_t r)
      : X(bf16(M, q.d_in)), A(bf16(r, q.d_in)), B(bf16(q.d_out, r)), Y(bf16(M, q.d_out)), T(bf16(M, r)),
        dY(bf16(M, q.d_out)), dX(bf16(M, q.d_in)), dA(bf16(r, q.d_in)), dB(bf16(q.d_out, r)) {}
};

void linear_paths() {
  struct Case {
    int64_t N, K, M;
    int32_t r;
    int dq;
  };
  const Case cases[] = {
      {4096, 4096, 1, 16, QLORA_DQ_E4M3},    // whole-row weight stream
      {6144, 4096, 2, 64, QLORA_DQ_E4M3},    // whole-row, two tokens
      {28672, 8192, 1, 64, QLORA_DQ_E4M3},   // weight stream
      {272, 320, 3, 8, QLORA_DQ_E4M3},       // split GEMV
      {4096, 4096, 16, 16, QLORA_DQ_E4M3},   // M = 16
      {512, 1024, 300, 16, QLORA_DQ_E4M3},   // fused mid-size GEMMs
      {1024, 2048, 2048, 16, QLORA_DQ_E4M3}, // decode once, split reduction
      {4096, 4096, 4096, 16, QLORA_DQ_E4M3}, // decode once
      {1040, 4096, 1, 24, QLORA_DQ_INT8},    // other formats decode once at every M
      {272, 320, 300, 8, QLORA_DQ_NONE},
  };
  for (const Case& c : cases) {
    Weight w(c.N, c.K, QLORA_CB_NF4, c.dq);
    Layer L(w.q, c.M, c.r);
    const size_t nf = ws_need(QLORA_OP_FWD, c.M, w.q, c.r), nb = ws_need(QLORA_OP_BWD, c.M, w.q, c.r);
    Buf wsf(nf), wsb(nb);
    uint16_t *X = L.X.as<uint16_t>(), *A = L.A.as<uint16_t>(), *B = L.B.as<uint16_t>();
    expect("fwd", QLORA_OK, [&] {
      return qlora_linear_fwd(&w.q, X, c.M, A, B, c.r, 32.f, L.Y.as<uint16_t>(), L.T.as<uint16_t>(), wsf.p, nf, nullptr);
    });
    expect("fwd no T", QLORA_OK, [&] {
      return qlora_linear_fwd(&w.q, X, c.M, A, B, c.r, 32.f, L.Y.as<uint16_t>(), nullptr, wsf.p, nf, nullptr);
    });
    expect("fwd small ws", QLORA_ERR_WORKSPACE, [&] {
      return qlora_linear_fwd(&w.q, X, c.M, A, B, c.r, 32.f, L.Y.as<uint16_t>(), nullptr, wsf.p, nf - 1, nullptr);
    });
    Buf wider(nf + 256);
    expect("fwd misaligned ws", QLORA_ERR_INVALID_ARG, [&] {
      return qlora_linear_fwd(&w.q, X, c.M, A, B, c.r, 32.f, L.Y.as<uint16_t>(), nullptr, wider.as<char>() + 8, nf,
                              nullptr);
    });
    expect("fwd misaligned X", QLORA_ERR_INVALID_ARG, [&] {
      return qlora_linear_fwd(&w.q, X + 1, c.M, A, B, c.r, 32.f, L.Y.as<uint16_t>(), nullptr, wsf.p, nf, nullptr);
    });
    expect("fwd alpha NaN", QLORA_ERR_INVALID_ARG, [&] {
      return qlora_linear_fwd(&w.q, X, c.M, A, B, c.r, NAN, L.Y.as<uint16_t>(), nullptr, wsf.p, nf, nullptr);
    });
    for (bool with_dx : {true, false})
      for (bool with_t : {true, false})
        expect("bwd", QLORA_OK, [&] {
          return qlora_linear_bwd(&w.q, X, L.dY.as<uint16_t>(), c.M, A, B, c.r, 32.f, with_t ? L.T.as<uint16_t>() : nullptr,
                                  with_dx ? L.dX.as<uint16_t>() : nullptr, L.dA.as<uint16_t>(), L.dB.as<uint16_t>(),
                                  wsb.p, nb, nullptr);
        });
    expect("bwd small ws", QLORA_ERR_WORKSPACE, [&] {
      return qlora_linear_bwd(&w.q, X, L.dY.as<uint16_t>(), c.M, A, B, c.r, 32.f, nullptr, L.dX.as<uint16_t>(),
                              L.dA.as<uint16_t>(), L.dB.as<uint16_t>(), wsb.p, nb - 1, nullptr);
    });
    expect("bwd null dA", QLORA_ERR_INVALID_ARG, [&] {
      return qlora_linear_bwd(&w.q, X, L.dY.as<uint16_t>(), c.M, A, B, c.r, 32.f, nullptr, L.dX.as<uint16_t>(),
                              nullptr, L.dB.as<uint16_t>(), wsb.p, nb, nullptr);
    });
    if (c.M <= 16 && c.dq == QLORA_DQ_E4M3 && nf <= QLORA_NOALLOC_SCRATCH_BYTES)
      expect("fwd noalloc", QLORA_OK, [&] {
        return qlora_linear_fwd_noalloc(&w.q, X, c.M, A, B, c.r, 32.f, L.Y.as<uint16_t>(), L.T.as<uint16_t>(), nullptr);
      });
  }
  // a forward whose workspace exceeds the fixed scratch is refused before any launch
  Weight big(4096, 4096);
  Layer L(big.q, 4096, 16);
  expect("noalloc beyond its scratch", QLORA_ERR_SCRATCH, [&] {
    return qlora_linear_fwd_noalloc(&big.q, L.X.as<uint16_t>(), 4096, L.A.as<uint16_t>(), L.B.as<uint16_t>(), 16, 32.f,
                                    L.Y.as<uint16_t>(), nullptr, nullptr);
  });
  Buf ws(ws_need(QLORA_OP_FWD, 1, big.q, 16));
  expect("workspace init", QLORA_OK, [&] { return qlora_workspace_init(ws.p, ws.n, nullptr); });
  expect("workspace init small", QLORA_ERR_WORKSPACE,
         [&] { return qlora_workspace_init(ws.p, QLORA_WS_COUNTER_BYTES - 1, nullptr); });
}

void grouped_paths() {
  for (int64_t M : {int64_t(1), int64_t(4), int64_t(300)}) {
    Weight q(8192, 4096), k(1024, 4096), v(1024, 4096);
    const qlora_nf4dq_t* W[3] = {&q.q, &k.q, &v.q};
    Layer a(q.q, M, 16), b(k.q, M, 16), c(v.q, M, 16);
    const uint16_t* A[3] = {a.A.as<uint16_t>(), b.A.as<uint16_t>(), c.A.as<uint16_t>()};
    const uint16_t* B[3] = {a.B.as<uint16_t>(), b.B.as<uint16_t>(), c.B.as<uint16_t>()};
    uint16_t* Y[3] = {a.Y.as<uint16_t>(), b.Y.as<uint16_t>(), c.Y.as<uint16_t>()};
    uint16_t* T[3] = {a.T.as<uint16_t>(), b.T.as<uint16_t>(), c.T.as<uint16_t>()};
    size_t need = 0;
    CHECK(qlora_workspace_size_multi(3, W, M, 16, &need) == QLORA_OK, "ws multi");
    Buf ws(need);
    expect("fwd multi", QLORA_OK,
           [&] { return qlora_linear_fwd_multi(3, W, a.X.as<uint16_t>(), M, A, B, 16, 32.f, Y, T, ws.p, need, nullptr); });
    expect("fwd multi small ws", QLORA_ERR_WORKSPACE, [&] {
      return qlora_linear_fwd_multi(3, W, a.X.as<uint16_t>(), M, A, B, 16, 32.f, Y, T, ws.p, need - 1, nullptr);
    });
    const uint16_t* Abad[3] = {A[0], nullptr, A[2]};
    expect("fwd multi null A", QLORA_ERR_INVALID_ARG, [&] {
      return qlora_linear_fwd_multi(3, W, a.X.as<uint16_t>(), M, Abad, B, 16, 32.f, Y, T, ws.p, need, nullptr);
    });
  }
}

void mlp_paths() {
  const int64_t d = 512, f = 1024;
  const int32_t r = 16;
  for (int64_t M : {int64_t(1), int64_t(64), int64_t(2048)}) {
    Weight g(f, d), u(f, d), dn(d, f);
    Buf X(bf16(M, d)), Y(bf16(M, d)), dY(bf16(M, d)), dX(bf16(M, d)), G(bf16(M, f)), U(bf16(M, f));
    Buf Ag(bf16(r, d)), Au(bf16(r, d)), Ad(bf16(r, f)), Bg(bf16(f, r)), Bu(bf16(f, r)), Bd(bf16(d, r));
    Buf dAg(bf16(r, d)), dAu(bf16(r, d)), dAd(bf16(r, f)), dBg(bf16(f, r)), dBu(bf16(f, r)), dBd(bf16(d, r));
    const uint16_t* A[3] = {Ag.as<uint16_t>(), Au.as<uint16_t>(), Ad.as<uint16_t>()};
    const uint16_t* B[3] = {Bg.as<uint16_t>(), Bu.as<uint16_t>(), Bd.as<uint16_t>()};
    uint16_t* dA[3] = {dAg.as<uint16_t>(), dAu.as<uint16_t>(), dAd.as<uint16_t>()};
    uint16_t* dB[3] = {dBg.as<uint16_t>(), dBu.as<uint16_t>(), dBd.as<uint16_t>()};
    size_t nf = 0, nb = 0;
    CHECK(qlora_mlp_workspace_size(QLORA_OP_FWD, M, &g.q, &u.q, &dn.q, r, &nf) == QLORA_OK, "mlp ws");
    CHECK(qlora_mlp_workspace_size(QLORA_OP_BWD, M, &g.q, &u.q, &dn.q, r, &nb) == QLORA_OK, "mlp ws");
    Buf wsf(nf), wsb(nb);
    expect("mlp fwd", QLORA_OK, [&] {
      return qlora_mlp_fwd(&g.q, &u.q, &dn.q, X.as<uint16_t>(), M, A, B, r, 32.f, Y.as<uint16_t>(), G.as<uint16_t>(),
                           U.as<uint16_t>(), wsf.p, nf, nullptr);
    });
    expect("mlp bwd", QLORA_OK, [&] {
      return qlora_mlp_bwd(&g.q, &u.q, &dn.q, X.as<uint16_t>(), dY.as<uint16_t>(), M, A, B, r, 32.f, G.as<uint16_t>(),
                           U.as<uint16_t>(), dX.as<uint16_t>(), dA, dB, wsb.p, nb, nullptr);
    });
    uint16_t* dBbad[3] = {dB[0], dB[1], nullptr};
    expect("mlp bwd null dB", QLORA_ERR_INVALID_ARG, [&] {
      return qlora_mlp_bwd(&g.q, &u.q, &dn.q, X.as<uint16_t>(), dY.as<uint16_t>(), M, A, B, r, 32.f, G.as<uint16_t>(),
                           U.as<uint16_t>(), dX.as<uint16_t>(), dA, dBbad, wsb.p, nb, nullptr);
    });
    expect("mlp fwd small ws", QLORA_ERR_WORKSPACE, [&] {
      return qlora_mlp_fwd(&g.q, &u.q, &dn.q, X.as<uint16_t>(), M, A, B, r, 32.f, Y.as<uint16_t>(), G.as<uint16_t>(),
                           U.as<uint16_t>(), wsf.p, nf - 1, nullptr);
    });
  }
}

void other_paths() {
  const int64_t n = 41943040 / 16 + 8;  // a ragged count
  Buf master(4 * n), m(4 * n), v(4 * n), grad(2 * n), param(2 * n);
  expect("adamw", QLORA_OK, [&] {
    return qlora_adamw_step(master.as<float>(), m.as<float>(), v.as<float>(), grad.as<uint16_t>(), param.as<uint16_t>(),
                            n, 1, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, nullptr);
  });
  expect("adamw step 0", QLORA_ERR_INVALID_ARG, [&] {
    return qlora_adamw_step(master.as<float>(), m.as<float>(), v.as<float>(), grad.as<uint16_t>(), param.as<uint16_t>(),
                            n, 0, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, nullptr);
  });
  Buf in(4 * 1001), out(1001);
  expect("e4m3", QLORA_OK, [&] { return qlora_e4m3_encode(in.as<float>(), out.as<uint8_t>(), 1001, nullptr); });
  // timing: events are created and read back through the stand-in
  CHECK(qlora_timing_enable((1 << QLORA_K_COUNT) - 1) == QLORA_OK, "timing enable");
  Weight w(4096, 4096);
  Layer L(w.q, 1, 16);
  const size_t nf = ws_need(QLORA_OP_FWD, 1, w.q, 16);
  Buf ws(nf);
  for (int i = 0; i < 3; ++i)
    expect("timed fwd", QLORA_OK, [&] {
      return qlora_linear_fwd(&w.q, L.X.as<uint16_t>(), 1, L.A.as<uint16_t>(), L.B.as<uint16_t>(), 16, 32.f,
                              L.Y.as<uint16_t>(), nullptr, ws.p, nf, nullptr);
    });
  for (int k = 0; k < QLORA_K_COUNT; ++k) {
    double ms = -1;
    int64_t launches = -1;
    CHECK(qlora_timing_read(k, &ms, &launches) == QLORA_OK, "timing read %d", k);
    CHECK(ms >= 0 && launches >= 0, "timing values");
  }
  CHECK(qlora_timing_enable(0) == QLORA_OK, "timing off");
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: %s FOLD_FILE\n", argv[0]);
    return 2;
  }
  fold(argv[1]);
  sizes();
  quantize_paths();
  linear_paths();
  grouped_paths();
  mlp_paths();
  other_paths();
  std::printf("launches %zu\n", sim::launches());
  std::printf("OK %d\n", g_checks);
  return 0;
}
