// Oracle for the block-scaled routed-expert MoE layer and the dense block-32
// FP8 projection.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
// CPU-baseline leg of the benchmark load this library; the product path never
// does, and this file shares no code, header or table with the HIP library.
//
// What it computes, and where the pages say so:
//   * "New Deepseek 4.1 flash recipe" (forum thread), post #6, "How it works":
//     routed experts with FP8 activations x FP4 weights; block-scaled MMAs for
//     MXFP8, FP8 x FP4 and MXFP4; dense MXFP8 projections.
//   * same post, "Why TileLang": the MoE top-k gate, SwiGLU and the
//     per-block FP8/FP4 quantization casts; every reduction in a fixed order.
//   * spark-ds41f README, "Current baseline": block-32 FP8 projections,
//     FP8 x FP4 routed experts, per-row results independent of the batch.
//   * same thread, post #2, "What changed": verification rows whose survival
//     estimate is below 0.2 skip the routed experts.
//   * DeepSeek-V4.1-Flash-4x-DGX-Spark-TP4 README, settings table, row
//     "Experts": a per-slot buffer summed in a fixed order instead of atomics.
// The pages never spell out the element and scale encodings; the MX prefix
// refers to the OCP Microscaling Formats v1.0 specification, whose E4M3, E2M1
// and E8M0 definitions are written out below.
//
// Arithmetic: every product of decoded operands is exact in double, every sum
// is accumulated in double in ascending index order, and results are rounded
// to fp32 where the method stores fp32.  Work is split over std::threads by
// independent outputs only, so the thread count never changes a result.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// ---------------------------------------------------------------- formats --
// OCP MX v1.0, FP8 E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits;
// exponent field 0 is subnormal; S.1111.111 is NaN; there is no infinity.
double e4m3_value(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return std::nan("");
  const double mag = (e == 0) ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

// OCP MX v1.0, FP4 E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit.
double e2m1_value(uint8_t n) {
  n &= 15;
  const int s = n >> 3, e = (n >> 1) & 3, m = n & 1;
  const double mag = (e == 0) ? m * 0.5 : std::ldexp(1.0 + m / 2.0, e - 1);
  return s ? -mag : mag;
}

// OCP MX v1.0, E8M0 scale: 2^(code - 127); code 255 is NaN.
double e8m0_value(uint8_t c) {
  if (c == 255) return std::nan("");
  return std::ldexp(1.0, int(c) - 127);
}

// Element i of a packed FP4 row: element 2j sits in the low nibble of byte j.
inline uint8_t fp4_nibble(const uint8_t* row, int64_t i) {
  const uint8_t b = row[i >> 1];
  return (i & 1) ? uint8_t(b >> 4) : uint8_t(b & 15);
}

// ----------------------------------------------------------- quantizer ----
// An element format as the set of its non-negative finite codes, sorted by
// value (both E4M3 and E2M1 codes grow monotonically with the magnitude).
struct Grid {
  std::vector<double> mag;  // magnitudes, ascending
  std::vector<uint8_t> code;
  int emax;                 // exponent of the largest normal (8 or 2)
  uint8_t sign_bit;
};

const Grid& grid_e4m3() {
  static const Grid g = [] {
    Grid r;
    for (int c = 0; c < 0x7F; ++c) { r.mag.push_back(e4m3_value(uint8_t(c))); r.code.push_back(uint8_t(c)); }
    r.emax = 8;  // 448 = 1.75 * 2^8
    r.sign_bit = 0x80;
    return r;
  }();
  return g;
}

const Grid& grid_e2m1() {
  static const Grid g = [] {
    Grid r;
    for (int c = 0; c < 8; ++c) { r.mag.push_back(e2m1_value(uint8_t(c))); r.code.push_back(uint8_t(c)); }
    r.emax = 2;  // 6 = 1.5 * 2^2
    r.sign_bit = 0x8;
    return r;
  }();
  return g;
}

// Shared scale of one block (OCP MX v1.0 conversion): X = 2^(floor(log2 amax) - emax),
// stored as the biased E8M0 code, clamped to the representable range; amax == 0 -> code 0.
uint8_t block_scale_code(const float* v, int n, int emax) {
  double amax = 0.0;
  for (int i = 0; i < n; ++i) amax = std::max(amax, std::fabs(double(v[i])));
  if (amax == 0.0) return 0;
  int ex = 0;
  std::frexp(amax, &ex);          // amax = f * 2^ex, f in [0.5, 1)  ->  floor(log2 amax) = ex - 1
  const int code = (ex - 1) - emax + 127;
  return uint8_t(std::min(254, std::max(0, code)));
}

// The finite grid value nearest to |t|; an exact tie goes to the even code;
// beyond the largest value the result saturates to it.  The sign is kept, so
// a negative input that rounds to zero becomes negative zero.
uint8_t round_to_grid(double t, bool negative, const Grid& g) {
  const double a = std::fabs(t);
  const auto& m = g.mag;
  size_t hi = std::lower_bound(m.begin(), m.end(), a) - m.begin();  // first mag >= a
  size_t best;
  if (hi == m.size()) {
    best = m.size() - 1;                 // above the largest finite value: saturate
  } else if (hi == 0 || m[hi] == a) {
    best = hi;
  } else {
    const size_t lo = hi - 1;
    const double dlo = a - m[lo], dhi = m[hi] - a;
    if (dlo < dhi) best = lo;
    else if (dhi < dlo) best = hi;
    else best = (g.code[lo] % 2 == 0) ? lo : hi;   // tie: even code
  }
  return uint8_t(g.code[best] | (negative ? g.sign_bit : 0));
}

// One block of n <= 32 values -> element codes and the scale code.
uint8_t quantize_block(const float* v, int n, const Grid& g, uint8_t* codes) {
  const uint8_t sc = block_scale_code(v, n, g.emax);
  const double X = e8m0_value(sc);
  for (int i = 0; i < n; ++i) codes[i] = round_to_grid(double(v[i]) / X, std::signbit(v[i]), g);
  return sc;
}

int resolve_threads(int threads) {
  if (threads > 0) return threads;
  const unsigned h = std::thread::hardware_concurrency();
  return h ? int(h) : 1;
}

// Run f(i) for i in [0, n) over `threads` workers, each taking a contiguous chunk.
template <class F>
void parallel_for(int64_t n, int threads, F f) {
  threads = int(std::min<int64_t>(resolve_threads(threads), std::max<int64_t>(n, 1)));
  if (threads <= 1) { for (int64_t i = 0; i < n; ++i) f(i); return; }
  std::vector<std::thread> pool;
  const int64_t chunk = (n + threads - 1) / threads;
  for (int w = 0; w < threads; ++w) {
    const int64_t b = w * chunk, e = std::min(n, b + chunk);
    if (b >= e) break;
    pool.emplace_back([=] { for (int64_t i = b; i < e; ++i) f(i); });
  }
  for (auto& t : pool) t.join();
}

// --------------------------------------------------------- the FFN pair ---
struct Layer {
  const uint8_t* x; const uint8_t* x_sc; int H;
  const uint8_t* w13; const uint8_t* w13_sc;
  const uint8_t* w2; const uint8_t* w2_sc; int I;
};

// Gate/up projection of token t through expert e: h[2I] (fp32), rows [0, I)
// of W13 are the gate, rows [I, 2I) the up projection.
void gate_up(const Layer& L, int t, int e, float* h) {
  const int H = L.H, I = L.I;
  std::vector<double> xv(H);
  const uint8_t* xr = L.x + int64_t(t) * H;
  const uint8_t* xs = L.x_sc + int64_t(t) * (H / 32);
  for (int k = 0; k < H; ++k) xv[k] = e4m3_value(xr[k]) * e8m0_value(xs[k / 32]);
  for (int n = 0; n < 2 * I; ++n) {
    const int64_t row = int64_t(e) * 2 * I + n;
    const uint8_t* wr = L.w13 + row * (H / 2);
    const uint8_t* ws = L.w13_sc + row * (H / 32);
    double acc = 0.0;
    for (int k = 0; k < H; ++k) acc += xv[k] * (e2m1_value(fp4_nibble(wr, k)) * e8m0_value(ws[k / 32]));
    h[n] = float(acc);
  }
}

// SwiGLU of h (a = silu(gate) * up, silu(g) = g / (1 + exp(-g)), in double,
// rounded to fp32), then the requant of the intermediate to FP8 E4M3 with one
// E8M0 scale per 32 values.  a_out (optional) receives the fp32 a.
void swiglu_requant(const float* h, int I, uint8_t* q, uint8_t* qsc, float* a_out) {
  std::vector<float> a(I);
  for (int i = 0; i < I; ++i) {
    const double g = h[i], u = h[I + i];
    a[i] = float(g / (1.0 + std::exp(-g)) * u);
  }
  for (int b = 0; b < I / 32; ++b) qsc[b] = quantize_block(&a[b * 32], 32, grid_e4m3(), &q[b * 32]);
  if (a_out) std::memcpy(a_out, a.data(), sizeof(float) * I);
}

// Down projection of one intermediate row (codes q, scales qsc) through expert e: o[H].
void down(const Layer& L, const uint8_t* q, const uint8_t* qsc, int e, float* o) {
  const int H = L.H, I = L.I;
  std::vector<double> av(I);
  for (int i = 0; i < I; ++i) av[i] = e4m3_value(q[i]) * e8m0_value(qsc[i / 32]);
  for (int n = 0; n < H; ++n) {
    const int64_t row = int64_t(e) * H + n;
    const uint8_t* wr = L.w2 + row * (I / 2);
    const uint8_t* ws = L.w2_sc + row * (I / 32);
    double acc = 0.0;
    for (int k = 0; k < I; ++k) acc += av[k] * (e2m1_value(fp4_nibble(wr, k)) * e8m0_value(ws[k / 32]));
    o[n] = float(acc);
  }
}

// One routed pair (token t, expert e): gate/up, SwiGLU, requant, down.
// Outputs o[H] and, when non-null, the diagnostics h[2I], a[I], q[I], q_sc[I/32].
void pair_ffn(const Layer& L, int t, int e, float* o, float* h_out, float* a_out, uint8_t* q_out, uint8_t* qsc_out) {
  const int I = L.I;
  std::vector<float> h(2 * I);
  std::vector<uint8_t> q(I), qsc(I / 32);
  gate_up(L, t, e, h.data());
  swiglu_requant(h.data(), I, q.data(), qsc.data(), a_out);
  down(L, q.data(), qsc.data(), e, o);
  if (h_out) std::memcpy(h_out, h.data(), sizeof(float) * 2 * I);
  if (q_out) std::memcpy(q_out, q.data(), I);
  if (qsc_out) std::memcpy(qsc_out, qsc.data(), I / 32);
}

// y_t = sum over slots j = 0..k-1 of w_tj * o_tj in double, rounded to fp32.
float combine(const float* w, const float* const* o, int k, int n) {
  double acc = 0.0;
  for (int j = 0; j < k; ++j)
    if (o[j]) acc += double(w[j]) * double(o[j][n]);
  return float(acc);
}

}  // namespace

extern "C" {

// ---- format decode (exported for the table tests) ----
double or_e4m3_value(uint8_t c) { return e4m3_value(c); }
double or_e2m1_value(uint8_t n) { return e2m1_value(n); }
double or_e8m0_value(uint8_t c) { return e8m0_value(c); }

// ---- quantizers: fp32 [rows][cols] -> codes + one scale per 32 along cols ----
// E4M3 codes are one byte each ([rows][cols]); E2M1 codes are packed two per
// byte ([rows][cols/2], element 2j in the low nibble).  cols % 32 == 0.
int or_quantize_e4m3(const float* v, int64_t rows, int64_t cols, uint8_t* q, uint8_t* sc, int threads) {
  if (cols % 32) return -1;
  parallel_for(rows, threads, [&](int64_t r) {
    for (int64_t b = 0; b < cols / 32; ++b)
      sc[r * (cols / 32) + b] = quantize_block(v + r * cols + b * 32, 32, grid_e4m3(), q + r * cols + b * 32);
  });
  return 0;
}

int or_quantize_e2m1(const float* v, int64_t rows, int64_t cols, uint8_t* q, uint8_t* sc, int threads) {
  if (cols % 32) return -1;
  parallel_for(rows, threads, [&](int64_t r) {
    uint8_t codes[32];
    for (int64_t b = 0; b < cols / 32; ++b) {
      sc[r * (cols / 32) + b] = quantize_block(v + r * cols + b * 32, 32, grid_e2m1(), codes);
      for (int j = 0; j < 16; ++j)
        q[r * (cols / 2) + b * 16 + j] = uint8_t(codes[2 * j] | (codes[2 * j + 1] << 4));
    }
  });
  return 0;
}

// Dequantize codes (fmt 0 = E4M3 bytes, 1 = packed E2M1) to double.
int or_dequantize(const uint8_t* q, const uint8_t* sc, int64_t rows, int64_t cols, int fmt, double* out) {
  if (cols % 32) return -1;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      const double s = e8m0_value(sc[r * (cols / 32) + c / 32]);
      const double v = fmt == 0 ? e4m3_value(q[r * cols + c]) : e2m1_value(fp4_nibble(q + r * (cols / 2), c));
      out[r * cols + c] = v * s;
    }
  return 0;
}

// ---- top-k gate and bucketing ----
// Per row: experts ordered by (logit descending, index ascending) under float
// comparison; the first k are slots 0..k-1.  Weights are the softmax over the
// selected logits, w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), in double,
// rounded to fp32.  A row is dead when survival != NULL and survival[t] <
// skip_below; dead rows keep their ids and weights but enter no bucket.
// Buckets list the live (t, j) pairs by expert ascending, then t ascending:
// perm[p] = t*k + j for p < P (then -1), slot_pos[t*k+j] = p (or -1),
// offsets[e] = first p of expert e, offsets[E] = P.
int or_route(const float* logits, int T, int E, int k, const float* survival, float skip_below,
             int32_t* ids, float* w, int32_t* offsets, int32_t* perm, int32_t* slot_pos) {
  if (T < 0 || E < 1 || k < 1 || k > E) return -1;
  std::vector<int> order(E);
  for (int t = 0; t < T; ++t) {
    const float* l = logits + int64_t(t) * E;
    for (int e = 0; e < E; ++e) order[e] = e;
    std::sort(order.begin(), order.end(), [l](int a, int b) {
      if (l[a] > l[b]) return true;
      if (l[b] > l[a]) return false;
      return a < b;
    });
    double den = 0.0;
    std::vector<double> ex(k);
    for (int j = 0; j < k; ++j) {
      ex[j] = std::exp(double(l[order[j]]) - double(l[order[0]]));
      den += ex[j];
    }
    for (int j = 0; j < k; ++j) {
      ids[int64_t(t) * k + j] = order[j];
      w[int64_t(t) * k + j] = float(ex[j] / den);
    }
  }
  int32_t p = 0;
  for (int64_t i = 0; i < int64_t(T) * k; ++i) { perm[i] = -1; slot_pos[i] = -1; }
  for (int e = 0; e < E; ++e) {
    offsets[e] = p;
    for (int t = 0; t < T; ++t) {
      if (survival && survival[t] < skip_below) continue;
      for (int j = 0; j < k; ++j)
        if (ids[int64_t(t) * k + j] == e) { perm[p] = t * k + j; slot_pos[int64_t(t) * k + j] = p; ++p; }
    }
  }
  offsets[E] = p;
  return 0;
}

// ---- top-k gate with router-live verification rows ----
// Verification rows that the confidence estimate does not expect to survive
// (survival[t] < reuse_below) reuse their anchor row's experts instead of
// skipping the experts: no weight is read that the anchor does not read, and
// the row still gets an output (DeepSeek-V4.1-Flash-4x-DGX-Spark-TP4 README,
// settings table, row "Verify length").  Read here as: such a row t with an
// anchor a = anchor[t] in [0, T), a != t, takes row a's own top-k experts in
// row a's slot order (whatever row a's survival), weighted by the softmax of
// row t's own logits over those experts, w_j = exp(l_j - m) / sum_i
// exp(l_i - m) with m the largest of them, in double, rounded to fp32.  Every
// other row keeps its own top-k.  Every pair of every row enters the buckets
// (same order as or_route).
int or_route_live(const float* logits, int T, int E, int k, const float* survival, float reuse_below,
                  const int32_t* anchor, int32_t* ids, float* w, int32_t* offsets, int32_t* perm,
                  int32_t* slot_pos) {
  if (T < 0 || E < 1 || k < 1 || k > E) return -1;
  std::vector<int32_t> own(int64_t(T) * k);
  std::vector<float> own_w(int64_t(T) * k);
  std::vector<int32_t> off(E + 1), pm(int64_t(T) * k), sp(int64_t(T) * k);
  if (or_route(logits, T, E, k, nullptr, 0.0f, own.data(), own_w.data(), off.data(), pm.data(), sp.data()))
    return -1;
  for (int t = 0; t < T; ++t) {
    const int a = anchor ? anchor[t] : t;
    const bool reuse = survival && survival[t] < reuse_below && a >= 0 && a < T && a != t;
    const int src = reuse ? a : t;
    const float* l = logits + int64_t(t) * E;
    double m = -INFINITY;
    for (int j = 0; j < k; ++j) m = std::max(m, double(l[own[int64_t(src) * k + j]]));
    std::vector<double> ex(k);
    double den = 0.0;
    for (int j = 0; j < k; ++j) {
      ex[j] = std::exp(double(l[own[int64_t(src) * k + j]]) - m);
      den += ex[j];
    }
    for (int j = 0; j < k; ++j) {
      ids[int64_t(t) * k + j] = own[int64_t(src) * k + j];
      w[int64_t(t) * k + j] = float(ex[j] / den);
    }
  }
  int32_t p = 0;
  for (int e = 0; e < E; ++e) {
    offsets[e] = p;
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j)
        if (ids[int64_t(t) * k + j] == e) { perm[p] = t * k + j; slot_pos[int64_t(t) * k + j] = p; ++p; }
  }
  offsets[E] = p;
  return 0;
}

// ---- routed-expert layer on a set of token rows ----
// For each row t listed in rows[0..nrows): if live[t], y_t = sum over slots j
// in order 0..k-1 of w_tj * o_tj (double, rounded to fp32), where o_tj is the
// pair output of expert ids[t][j]; dead rows are +0.  y is [nrows][H].
int or_moe_rows(const uint8_t* x, const uint8_t* x_sc, int H,
                const int32_t* ids, const float* w, const uint8_t* live, int k,
                const uint8_t* w13, const uint8_t* w13_sc, const uint8_t* w2, const uint8_t* w2_sc,
                int E, int I, const int32_t* rows, int nrows, float* y, int threads) {
  if (H % 32 || I % 32 || k < 1 || E < 1) return -1;
  const Layer L{x, x_sc, H, w13, w13_sc, w2, w2_sc, I};
  // pair outputs first (one thread per pair), then the fixed-order combine.
  std::vector<float> o(int64_t(nrows) * k * H, 0.0f);
  parallel_for(int64_t(nrows) * k, threads, [&](int64_t idx) {
    const int r = int(idx / k), j = int(idx % k);
    const int t = rows[r];
    if (!live[t]) return;
    pair_ffn(L, t, ids[int64_t(t) * k + j], &o[idx * H], nullptr, nullptr, nullptr, nullptr);
  });
  parallel_for(nrows, threads, [&](int64_t r) {
    const int t = rows[r];
    std::vector<const float*> op(k);
    for (int j = 0; j < k; ++j) op[j] = live[t] ? &o[(r * k + j) * H] : nullptr;
    for (int n = 0; n < H; ++n) y[r * H + n] = live[t] ? combine(w + int64_t(t) * k, op.data(), k, n) : 0.0f;
  });
  return 0;
}

// The second half of the layer from a given FP8 intermediate: q [P][I] and
// q_sc [P][I/32] indexed by bucket position p (slot_pos[t][j] = p, -1 when the
// pair is dead).  o_tj = down(q[p]) and y_t as in or_moe_rows.  y [nrows][H].
int or_down_combine(const uint8_t* q, const uint8_t* q_sc, const int32_t* slot_pos, const int32_t* ids,
                    const float* w, int k, const uint8_t* w2, const uint8_t* w2_sc, int H, int E, int I,
                    const int32_t* rows, int nrows, float* y, int threads) {
  if (H % 32 || I % 32 || k < 1 || E < 1) return -1;
  const Layer L{nullptr, nullptr, H, nullptr, nullptr, w2, w2_sc, I};
  std::vector<float> o(int64_t(nrows) * k * H, 0.0f);
  parallel_for(int64_t(nrows) * k, threads, [&](int64_t idx) {
    const int r = int(idx / k), j = int(idx % k);
    const int t = rows[r];
    const int p = slot_pos[int64_t(t) * k + j];
    if (p < 0) return;
    down(L, q + int64_t(p) * I, q_sc + int64_t(p) * (I / 32), ids[int64_t(t) * k + j], &o[idx * H]);
  });
  parallel_for(nrows, threads, [&](int64_t r) {
    const int t = rows[r];
    std::vector<const float*> op(k);
    for (int j = 0; j < k; ++j) op[j] = slot_pos[int64_t(t) * k + j] >= 0 ? &o[(r * k + j) * H] : nullptr;
    for (int n = 0; n < H; ++n) y[r * H + n] = combine(w + int64_t(t) * k, op.data(), k, n);
  });
  return 0;
}

// SwiGLU + requant of given fp32 gate/up rows h [n][2I] -> q [n][I], q_sc [n][I/32], a [n][I].
int or_swiglu_requant(const float* h, int64_t n, int I, uint8_t* q, uint8_t* q_sc, float* a) {
  if (I % 32) return -1;
  for (int64_t r = 0; r < n; ++r)
    swiglu_requant(h + r * 2 * I, I, q + r * I, q_sc + r * (I / 32), a ? a + r * I : nullptr);
  return 0;
}

// Gate/up values of n (token, expert) pairs, one thread per pair: h [n][2I],
// row i = gate_up(ts[i], es[i]) (diagnostics of the gate/up GEMM alone).
int or_gate_up_pairs(const uint8_t* x, const uint8_t* x_sc, int H, const int32_t* ts, const int32_t* es, int n,
                     const uint8_t* w13, const uint8_t* w13_sc, int I, float* h, int threads) {
  if (H % 32 || I % 32 || n < 0) return -1;
  const Layer L{x, x_sc, H, w13, w13_sc, nullptr, nullptr, I};
  parallel_for(n, threads, [&](int64_t i) { gate_up(L, ts[i], es[i], h + i * 2 * I); });
  return 0;
}

// One pair with its intermediates (diagnostics): h[2I], a[I], q[I], q_sc[I/32], o[H].
int or_pair_ffn(const uint8_t* x, const uint8_t* x_sc, int H, int t, int e,
                const uint8_t* w13, const uint8_t* w13_sc, const uint8_t* w2, const uint8_t* w2_sc, int I,
                float* h, float* a, uint8_t* q, uint8_t* q_sc, float* o) {
  if (H % 32 || I % 32) return -1;
  const Layer L{x, x_sc, H, w13, w13_sc, w2, w2_sc, I};
  pair_ffn(L, t, e, o, h, a, q, q_sc);
  return 0;
}

// ---- dense block-32 FP8 GEMM: y[m][n] = sum_k a[m][k] w[n][k] (decoded), fp32 out ----
// Only the rows listed in rows[0..nrows) are computed; y is [nrows][N].
int or_block_gemm(const uint8_t* a, const uint8_t* a_sc, const uint8_t* wq, const uint8_t* w_sc,
                  int N, int K, const int32_t* rows, int nrows, float* y, int threads) {
  if (K % 32) return -1;
  parallel_for(int64_t(nrows) * N, threads, [&](int64_t idx) {
    const int64_t r = idx / N, n = idx % N;
    const int64_t m = rows[r];
    double acc = 0.0;
    for (int64_t kk = 0; kk < K; ++kk) {
      const double av = e4m3_value(a[m * K + kk]) * e8m0_value(a_sc[m * (K / 32) + kk / 32]);
      const double wv = e4m3_value(wq[n * K + kk]) * e8m0_value(w_sc[n * (K / 32) + kk / 32]);
      acc += av * wv;
    }
    y[idx] = float(acc);
  });
  return 0;
}

// ---- router logits ----
// The routed experts are picked from one score per (row, expert): the
// hidden row against that expert's gate row, a linear map without bias
// (post #6 "How it works": the MoE top-k gate; "Kernel by kernel against
// B12X": the router's own time per step).  The pages give no precisions;
// read here as bf16 hidden states and bf16 gate rows, accumulated exactly
// and stored as fp32 logits.
//   logits[r][e] = fp32( sum_{j=0..H-1} h[rows[r]][j] * wg[e][j] )
// bf16 is the upper half of an IEEE binary32, so decoding is exact.
static double bf16_value(uint16_t b) {
  const uint32_t u = uint32_t(b) << 16;
  float f; std::memcpy(&f, &u, 4);
  return double(f);
}

int or_router_logits(const uint16_t* h, const uint16_t* wg, int E, int H, const int32_t* rows, int nrows,
                     float* logits, int threads) {
  if (E < 1 || H < 1) return -1;
  parallel_for(int64_t(nrows) * E, threads, [&](int64_t idx) {
    const int64_t r = idx / E, e = idx % E;
    const int64_t m = rows[r];
    double acc = 0.0;
    for (int64_t j = 0; j < H; ++j) acc += bf16_value(h[m * H + j]) * bf16_value(wg[e * H + j]);
    logits[idx] = float(acc);
  });
  return 0;
}

// ---- fp32 -> bf16, round to nearest, ties to even (finite inputs) ----
// The two bf16 neighbours of v are its truncation and the next bf16 value
// away from zero; the nearer one wins, an exact tie takes the even one.
void or_f32_to_bf16(const float* v, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t bits; std::memcpy(&bits, &v[i], 4);
    const uint32_t lo = bits & 0xFFFF0000u, hi = lo + 0x10000u;
    float flo, fhi; std::memcpy(&flo, &lo, 4); std::memcpy(&fhi, &hi, 4);
    const double dlo = std::fabs(double(v[i]) - double(flo)), dhi = std::fabs(double(fhi) - double(v[i]));
    uint32_t pick;
    if (dlo < dhi) pick = lo;
    else if (dhi < dlo) pick = hi;
    else pick = ((lo >> 16) & 1) ? hi : lo;
    out[i] = uint16_t(pick >> 16);
  }
}

int or_hardware_threads(void) { return resolve_threads(0); }

}  // extern "C"
