// Host half of libtq.so: seeded rotation and sketch, Lloyd-Max codebook,
// device tables, argument validation and the C ABI entry points.
//
// Method: noze.it, "TurboQuant-MLX: quantizzare pesi e KV cache per LLM
// open-weight su Mac", sections "Il metodo TurboQuant, in breve" (random
// rotation, per-coordinate optimal scalar quantizer, 1-bit JL sketch of the
// residual) and "Cosa aggiunge turboquant-mlx" (Lloyd-Max codebook).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "tq_internal.h"

namespace {

thread_local std::string g_err;

tq_status fail(tq_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

// ---------------------------------------------------------------------------
// Random streams.  SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): the state
// advances by 0x9E3779B97F4A7C15 and each output is the 64-bit finalizer of
// the new state.  Uniform doubles use the top 53 bits; Gaussians use
// Box-Muller on consecutive pairs, r = sqrt(-2 ln(1-u_a)) times cos then sin
// of 2 pi u_b, filled in order.

struct SplitMix64 {
  uint64_t state;
  uint64_t next() {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
};

double unit_double(uint64_t z) { return static_cast<double>(z >> 11) * 0x1.0p-53; }

void gaussian_fill(uint64_t seed, double* out, size_t n) {
  SplitMix64 g{seed};
  for (size_t i = 0; i < n; i += 2) {
    const double ua = unit_double(g.next());
    const double ub = unit_double(g.next());
    const double r = std::sqrt(-2.0 * std::log(1.0 - ua));
    const double ang = 2.0 * M_PI * ub;
    out[i] = r * std::cos(ang);
    if (i + 1 < n) out[i + 1] = r * std::sin(ang);
  }
}

// ---------------------------------------------------------------------------
// Haar rotation: Householder QR of the seeded Gaussian matrix A (row-major),
// A = Q R, then pi = Q diag(sign R_kk) so that the triangular factor has a
// positive diagonal (Mezzadri 2007), which makes pi unique.

void rotation_build(int d, uint64_t seed, double* pi) {
  std::vector<double> a(static_cast<size_t>(d) * d);
  gaussian_fill(seed, a.data(), a.size());
  std::vector<double> vs(static_cast<size_t>(d) * d, 0.0);  // Householder vectors, row k = v_k
  std::vector<double> vn(d, 0.0);                           // |v_k|^2 (0: identity reflector)
  std::vector<double> rdiag(d, 0.0);
  for (int k = 0; k < d; ++k) {
    double nrm2 = 0.0;
    for (int i = k; i < d; ++i) nrm2 += a[i * d + k] * a[i * d + k];
    const double nrm = std::sqrt(nrm2);
    if (nrm == 0.0) { rdiag[k] = 0.0; continue; }
    const double alpha = a[k * d + k] > 0 ? -nrm : nrm;  // R_kk after the reflection
    double* v = &vs[static_cast<size_t>(k) * d];
    for (int i = k; i < d; ++i) v[i] = a[i * d + k];
    v[k] -= alpha;
    double v2 = 0.0;
    for (int i = k; i < d; ++i) v2 += v[i] * v[i];
    vn[k] = v2;
    if (v2 == 0.0) { rdiag[k] = alpha; continue; }
    for (int j = k; j < d; ++j) {
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += v[i] * a[i * d + j];
      const double f = 2.0 * dot / v2;
      for (int i = k; i < d; ++i) a[i * d + j] -= f * v[i];
    }
    rdiag[k] = a[k * d + k];
  }
  // Q = H_0 H_1 ... H_{d-1}, accumulated by applying the reflectors to I from the left
  // in reverse order.
  std::vector<double> q(static_cast<size_t>(d) * d, 0.0);
  for (int i = 0; i < d; ++i) q[i * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    if (vn[k] == 0.0) continue;
    const double* v = &vs[static_cast<size_t>(k) * d];
    for (int j = 0; j < d; ++j) {
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += v[i] * q[i * d + j];
      const double f = 2.0 * dot / vn[k];
      for (int i = k; i < d; ++i) q[i * d + j] -= f * v[i];
    }
  }
  for (int i = 0; i < d; ++i)
    for (int k = 0; k < d; ++k) pi[i * d + k] = q[i * d + k] * (rdiag[k] < 0 ? -1.0 : 1.0);
}

// Randomized Hadamard rotation: pi = H diag(sigma) / sqrt(d), with the Sylvester
// Hadamard matrix H (entry (i, k) = (-1)^popcount(i & k)) and sigma_k the sign
// given by bit 63 of the k-th SplitMix64 output.

void hadamard_rotation_build(int d, uint64_t seed, double* pi) {
  SplitMix64 g{seed};
  std::vector<double> sigma(d);
  for (int k = 0; k < d; ++k) sigma[k] = (g.next() >> 63) ? -1.0 : 1.0;
  const double scale = 1.0 / std::sqrt(static_cast<double>(d));
  for (int i = 0; i < d; ++i)
    for (int k = 0; k < d; ++k) pi[i * d + k] = (__builtin_popcount(i & k) & 1 ? -scale : scale) * sigma[k];
}

// ---------------------------------------------------------------------------
// Lloyd-Max codebook for the law of one coordinate X of a uniform unit vector
// in R^d: density K_d (1-x^2)^((d-3)/2) on [-1, 1], i.e. (1+X)/2 ~
// Beta(a, a) with a = (d-1)/2.  Cell masses use the regularised incomplete
// beta function (continued fraction, DLMF 8.17.22, evaluated with the
// modified Lentz method); first moments have the closed form
// K_d/(d-1) [(1-lo^2)^((d-1)/2) - (1-hi^2)^((d-1)/2)].

double beta_cf(double a, double b, double x) {
  const double tiny = 1e-300;
  double c = 1.0, dd = 1.0 - (a + b) * x / (a + 1.0);
  if (std::fabs(dd) < tiny) dd = tiny;
  dd = 1.0 / dd;
  double h = dd;
  for (int m = 1; m <= 100000; ++m) {
    const double m2 = 2.0 * m;
    double num = m * (b - m) * x / ((a + m2 - 1.0) * (a + m2));
    dd = 1.0 + num * dd;
    if (std::fabs(dd) < tiny) dd = tiny;
    c = 1.0 + num / c;
    if (std::fabs(c) < tiny) c = tiny;
    dd = 1.0 / dd;
    h *= dd * c;
    num = -(a + m) * (a + b + m) * x / ((a + m2) * (a + m2 + 1.0));
    dd = 1.0 + num * dd;
    if (std::fabs(dd) < tiny) dd = tiny;
    c = 1.0 + num / c;
    if (std::fabs(c) < tiny) c = tiny;
    dd = 1.0 / dd;
    const double step = dd * c;
    h *= step;
    if (std::fabs(step - 1.0) < 1e-16) break;
  }
  return h;
}

// Regularised incomplete beta I_x(a, b).
double ibeta(double a, double b, double x) {
  if (x <= 0.0) return 0.0;
  if (x >= 1.0) return 1.0;
  const double lfront = std::lgamma(a + b) - std::lgamma(a) - std::lgamma(b) + a * std::log(x) +
                         b * std::log1p(-x);
  const double front = std::exp(lfront);
  if (x < (a + 1.0) / (a + b + 2.0)) return front * beta_cf(a, b, x) / a;
  return 1.0 - front * beta_cf(b, a, 1.0 - x) / b;
}

struct CoordLaw {
  int d;
  double a;       // (d-1)/2
  double kd;      // normaliser K_d
  explicit CoordLaw(int d_) : d(d_), a(0.5 * (d_ - 1)) {
    kd = std::exp(std::lgamma(0.5 * d_) - std::lgamma(0.5 * (d_ - 1))) / std::sqrt(M_PI);
  }
  double upper_tail(double x) const {  // P(X > x)
    if (x <= -1.0) return 1.0;
    if (x >= 1.0) return 0.0;
    return ibeta(a, a, 0.5 * (1.0 - x));
  }
  double mass(double lo, double hi) const { return upper_tail(lo) - upper_tail(hi); }
  double density(double x) const {
    const double t = 1.0 - x * x;
    return t <= 0.0 ? 0.0 : kd * std::pow(t, 0.5 * (d - 3));
  }
  double moment(double lo, double hi) const {
    const double p = 0.5 * (d - 1);
    auto g = [p](double x) { const double t = 1.0 - x * x; return t <= 0.0 ? 0.0 : std::pow(t, p); };
    return kd / (d - 1) * (g(lo) - g(hi));
  }
};

void codebook_build(int d, int bits, double* cen, double* bnd) {
  const CoordLaw law(d);
  const int L = 1 << bits;
  std::vector<double> c(L), t(L - 1), e(L + 1);
  // Start: conditional means of L equal-mass cells (quantiles by bisection).
  for (int j = 1; j < L; ++j) {
    const double target = 1.0 - static_cast<double>(j) / L;  // upper-tail mass above the edge
    double lo = -1.0, hi = 1.0;
    for (int it = 0; it < 200; ++it) {
      const double mid = 0.5 * (lo + hi);
      if (law.upper_tail(mid) > target) lo = mid; else hi = mid;
    }
    e[j] = 0.5 * (lo + hi);
  }
  e[0] = -1.0;
  e[L] = 1.0;
  for (int j = 0; j < L; ++j) c[j] = law.moment(e[j], e[j + 1]) / law.mass(e[j], e[j + 1]);
  double best = INFINITY;
  int stall = 0;
  // Above 16 levels the Lloyd map contracts slowly (tens of thousands of
  // steps at 256 levels): a few hundred steps, then Newton below.
  const int lloyd_steps = L > 16 ? 300 : 200000;
  for (int it = 0; it < lloyd_steps; ++it) {
    for (int j = 1; j < L; ++j) e[j] = 0.5 * (c[j - 1] + c[j]);
    std::vector<double> cn(L);
    for (int j = 0; j < L; ++j) cn[j] = law.moment(e[j], e[j + 1]) / law.mass(e[j], e[j + 1]);
    double step = 0.0;
    for (int j = 0; j < L; ++j) {
      const double sym = 0.5 * (cn[j] - cn[L - 1 - j]);  // the law is symmetric about 0
      step = std::fmax(step, std::fabs(sym - c[j]));
      c[j] = sym;
    }
    if (step < 1e-15) break;
    if (step < best) { best = step; stall = 0; }
    else if (++stall > 50 && step < 1e-13) break;
  }
  if (L > 16) {
    // Newton on the fixed-point conditions G_k = e_k - (c_{k-1} + c_k) / 2 = 0
    // over the interior edges e_1 .. e_{L-1}, c_j the centroid of [e_j,
    // e_{j+1}].  With P_j the cell mass and f the density,
    // dc_j/de_{j+1} = f(e_{j+1}) (e_{j+1} - c_j) / P_j and
    // dc_j/de_j = f(e_j) (c_j - e_j) / P_j, so the Jacobian is tridiagonal
    // (Thomas algorithm); steps are halved while they do not reduce max |G|.
    for (int j = 1; j < L; ++j) e[j] = 0.5 * (c[j - 1] + c[j]);
    std::vector<double> P(L), G(L), lo_d(L), di(L), up_d(L), rhs(L), en(L + 1);
    auto eval = [&](const std::vector<double>& ed, std::vector<double>& cc, std::vector<double>& pp,
                    std::vector<double>& gg) {
      double gmax = 0.0;
      for (int j = 0; j < L; ++j) {
        pp[j] = law.mass(ed[j], ed[j + 1]);
        cc[j] = law.moment(ed[j], ed[j + 1]) / pp[j];
      }
      for (int k = 1; k < L; ++k) {
        gg[k] = ed[k] - 0.5 * (cc[k - 1] + cc[k]);
        gmax = std::fmax(gmax, std::fabs(gg[k]));
      }
      return gmax;
    };
    std::vector<double> cc(L), pp(L), gg(L);
    double g = eval(e, c, P, G);
    for (int it = 0; it < 50 && g > 1e-17; ++it) {
      for (int k = 1; k < L; ++k) {
        const double fk = law.density(e[k]);
        di[k] = 1.0 - 0.5 * fk * ((e[k] - c[k - 1]) / P[k - 1] + (c[k] - e[k]) / P[k]);
        lo_d[k] = k > 1 ? -0.5 * law.density(e[k - 1]) * (c[k - 1] - e[k - 1]) / P[k - 1] : 0.0;
        up_d[k] = k < L - 1 ? -0.5 * law.density(e[k + 1]) * (e[k + 1] - c[k]) / P[k] : 0.0;
        rhs[k] = G[k];
      }
      for (int k = 2; k < L; ++k) {  // forward elimination
        const double m = lo_d[k] / di[k - 1];
        di[k] -= m * up_d[k - 1];
        rhs[k] -= m * rhs[k - 1];
      }
      rhs[L - 1] /= di[L - 1];
      for (int k = L - 2; k >= 1; --k) rhs[k] = (rhs[k] - up_d[k] * rhs[k + 1]) / di[k];
      double lam = 1.0, gn = INFINITY;
      for (int h = 0; h < 30; ++h, lam *= 0.5) {
        en = e;
        for (int k = 1; k < L; ++k) en[k] = e[k] - lam * rhs[k];
        bool ordered = true;
        for (int k = 0; k < L; ++k) ordered = ordered && en[k] < en[k + 1];
        if (!ordered) continue;
        gn = eval(en, cc, pp, gg);
        if (gn < g) break;
      }
      if (!(gn < g)) break;  // at the rounding floor
      e = en;
      c = cc;
      P = pp;
      G = gg;
      g = gn;
    }
    for (int j = 0; j < L; ++j) cc[j] = 0.5 * (c[j] - c[L - 1 - j]);  // the law is symmetric about 0
    c = cc;
  }
  for (int j = 0; j < L - 1; ++j) t[j] = 0.5 * (c[j] + c[j + 1]);
  if (L % 2 == 0) t[L / 2 - 1] = 0.0;
  std::memcpy(cen, c.data(), sizeof(double) * L);
  std::memcpy(bnd, t.data(), sizeof(double) * (L - 1));
}

// ---------------------------------------------------------------------------
// IEEE binary16 from a double, round to nearest even, in one rounding step.
uint16_t to_half(double v) {
  const uint16_t sign = std::signbit(v) ? 0x8000u : 0u;
  const double a = std::fabs(v);
  if (std::isnan(v)) return 0x7E00u;
  if (a >= 65520.0) return sign | 0x7C00u;
  if (a < 0x1.0p-14) {  // subnormal range: multiples of 2^-24
    const double m = std::nearbyint(a * 0x1.0p24);
    return sign | static_cast<uint16_t>(m);  // m == 1024 encodes the smallest normal
  }
  int e;
  std::frexp(a, &e);  // a = f 2^e, f in [0.5, 1)
  int ex = e - 1;     // a = 1.m 2^ex
  double m = std::nearbyint(std::ldexp(a, 10 - ex));  // in [1024, 2048]
  if (m >= 2048.0) { m = 1024.0; ++ex; }
  if (ex > 15) return sign | 0x7C00u;
  return sign | static_cast<uint16_t>(((ex + 15) << 10) | (static_cast<int>(m) - 1024));
}

// The value of a binary16 bit pattern (finite).
double from_half(uint16_t h) {
  const int ex = (h >> 10) & 31, m = h & 1023;
  const double a = ex == 0 ? std::ldexp(static_cast<double>(m), -24) : std::ldexp(1024.0 + m, ex - 25);
  return (h & 0x8000u) ? -a : a;
}

// Scale s in [1, 2) of a codebook's fp16 centroids: the kernels' lookup
// tables hold fp16(c_j s), and s is divided out in fp32 on the other operand
// (the query's coordinates before their hi + lo split, the value
// accumulator before the inverse rotation).  s minimises the largest relative
// rounding error over the centroids, searched over s = 1 + k / 2^16: for a
// 4-bit codebook that is about 4 times below the 2^-12 bound of plain fp16,
// more for fewer levels.  A pure function of the centroids.
double centroid_scale(const double* c, int n) {
  double best = INFINITY, best_s = 1.0;
  for (int k = 0; k < (1 << 16); ++k) {
    const double sc = 1.0 + k * 0x1.0p-16;
    double worst = 0.0;
    for (int j = 0; j < n && worst < best; ++j) {
      if (c[j] == 0.0) continue;
      const double v = c[j] * sc;
      worst = std::max(worst, std::fabs(from_half(to_half(v)) - v) / std::fabs(v));
    }
    if (worst < best) {
      best = worst;
      best_s = sc;
    }
  }
  return best_s;
}

// bfloat16 from a double, round to nearest even (one rounding step; finite
// values below the overflow threshold).
uint16_t to_bf16(double v) {
  if (v == 0.0) return std::signbit(v) ? 0x8000u : 0u;
  const uint16_t sign = std::signbit(v) ? 0x8000u : 0u;
  const double a = std::fabs(v);
  int e;
  std::frexp(a, &e);   // a = f 2^e, f in [0.5, 1)
  int ex = e - 1;      // a = 1.m 2^ex
  if (ex < -126) {     // subnormal: multiples of 2^-133
    const double m = std::nearbyint(std::ldexp(a, 133));
    return sign | static_cast<uint16_t>(m);
  }
  double m = std::nearbyint(std::ldexp(a, 7 - ex));  // in [128, 256]
  if (m >= 256.0) { m = 128.0; ++ex; }
  if (ex > 127) return sign | 0x7F80u;
  return sign | static_cast<uint16_t>(((ex + 127) << 7) | (static_cast<int>(m) - 128));
}

double from_bf16(uint16_t b) {
  const uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// ---------------------------------------------------------------------------
tq_status check_spec(const tq_spec* s, tq::Spec* out) {
  if (!s) return fail(TQ_E_ARG, "spec is NULL");
  if (s->d != TQ_DIM) return fail(TQ_E_UNSUPPORTED, "d must be 128");
  if (s->bits_lo == 8) {
    // 8-bit keys: uniform width, record layout, no sketch
    if (s->split != 128 || s->layout != TQ_LAYOUT_RECORD || s->qjl_m != 0)
      return fail(TQ_E_UNSUPPORTED, "8-bit codes need split 128, the record layout and no sketch");
  }
  auto okb = [](int b) { return b >= 2 && b <= 4; };
  if (!okb(s->bits_lo) && s->bits_lo != 8) return fail(TQ_E_UNSUPPORTED, "bits_lo must be 2, 3, 4 or 8");
  if (s->split != 64 && s->split != 128) return fail(TQ_E_UNSUPPORTED, "split must be 64 or 128");
  const int bhi = s->split == 128 ? s->bits_lo : s->bits_hi;
  if (!okb(bhi) && bhi != 8) return fail(TQ_E_UNSUPPORTED, "bits_hi must be 2, 3 or 4");
  const int bl = s->bits_lo;
  const bool combo_ok = (bl == bhi) || (bl == 4 && bhi == 3) || (bl == 3 && bhi == 2);
  if (!combo_ok) return fail(TQ_E_UNSUPPORTED, "mixed widths supported: 4/3 and 3/2 (split 64)");
  if (s->layout != TQ_LAYOUT_RECORD && s->layout != TQ_LAYOUT_TILED)
    return fail(TQ_E_ARG, "layout must be TQ_LAYOUT_RECORD or TQ_LAYOUT_TILED");
  if (s->qjl_m != 0 && s->qjl_m != TQ_QJL_M) return fail(TQ_E_UNSUPPORTED, "qjl_m must be 0 or 128");
  if (s->qjl_m && s->layout != TQ_LAYOUT_RECORD)
    return fail(TQ_E_UNSUPPORTED, "the QJL sketch needs the record layout");
  if (s->rotation != TQ_ROT_HAAR && s->rotation != TQ_ROT_HADAMARD && s->rotation != TQ_ROT_HADAMARD_FWHT)
    return fail(TQ_E_ARG, "rotation must be TQ_ROT_HAAR, TQ_ROT_HADAMARD or TQ_ROT_HADAMARD_FWHT");
  if (s->norm_f16 != 0 && s->norm_f16 != 1) return fail(TQ_E_ARG, "norm_f16 must be 0 or 1");
  if (out) {
    out->bits_lo = bl;
    out->bits_hi = bhi;
    out->qjl_m = s->qjl_m;
    out->layout = s->layout;
    out->code_bytes = 8 * (bl + bhi);
    out->norm16 = s->norm_f16;
    out->rotation = s->rotation;
  }
  return TQ_OK;
}

tq_status check_tables(const void* tables, const tq::Spec& sp, const char* what) {
  if (!tables) return fail(TQ_E_ARG, std::string(what) + " tables pointer is NULL");
  if (reinterpret_cast<uintptr_t>(tables) % 256)
    return fail(TQ_E_ARG, std::string(what) + " tables must be 256-byte aligned");
  (void)sp;
  return TQ_OK;
}

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

tq_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return TQ_OK;
  return fail(TQ_E_HIP, std::string(where) + ": " + hipGetErrorString(e));
}


// Cell tables of a codebook (fp32 boundaries, ascending): entry c = {bits of
// the one boundary inside cell c (or of +inf), number of boundaries below the
// cell}, so that the code of y in cell c is below + (y > boundary).  Cell c is
// the half-open interval [lo(c), lo(c + 1)); false when a cell holds two
// boundaries or a boundary lies less than `margin` below an upper edge.
template <class Lo>
bool cell_table(const float* bnd, int nb, uint32_t (*cell)[2], int entries, Lo lo_of, double margin) {
  for (int c = 0; c < entries; ++c) {
    const double lo = lo_of(c), hi = lo_of(c + 1);
    uint32_t below = 0, inside = 0;
    float b_in = INFINITY;
    for (int j = 0; j < nb; ++j) {
      const double t = bnd[j];
      if (t < lo) ++below;
      else if (t < hi) {
        ++inside;
        b_in = bnd[j];
      }
      if (t < lo && lo - t < margin) return false;
    }
    if (inside > 1) return false;
    uint32_t bits;
    std::memcpy(&bits, &b_in, 4);
    cell[c][0] = bits;
    cell[c][1] = below;
  }
  return true;
}

// 2- to 4-bit codebooks: the kernels take the cell of y from the fp32 fma
// u = fl(512 y + 512 + 2^23), one rounding to nearest even, as bits 3..10 of
// u's mantissa, i.e. c = RNE(512 y + 512) >> 3.  Ties go to even integers, so
// cell c is exactly [(8c - 1/2) / 512 - 1, (8c + 15/2) / 512 - 1) for every
// |y| <= 1 + 1/1024, and the code below + (y > boundary) is exact with no
// margin.
bool cell_table_u(const float* bnd, int nb, uint32_t (*cell)[2]) {
  return cell_table(bnd, nb, cell, tq::CELL_ENTRIES, [](int c) { return (8.0 * c - 0.5) / 512.0 - 1.0; }, 0.0);
}

// 8-bit codebooks: cell c = [c / 1024 - 1/2, (c + 1) / 1024 - 1/2), found as
// the truncated fp32 fma(y, 1024, 512) clamped to [0, 1024], which can move a
// y lying just below an edge up into the next cell (by at most 2^-25): no
// boundary may lie within 1e-7 below an edge.
bool cell_table_8(const float* bnd, int nb, uint32_t (*cell)[2]) {
  return cell_table(bnd, nb, cell, tq::CELL8_ENTRIES, [](int c) { return c / 1024.0 - 0.5; }, 1e-7);
}

}  // namespace

extern "C" {

int32_t tq_format_version(void) { return TQ_FORMAT_VERSION; }

const char* tq_last_error(void) { return g_err.c_str(); }

tq_status tq_codebook_build(int32_t d, int32_t bits, double* centroids, double* boundaries) {
  if (d < 3 || d > 65536) return fail(TQ_E_ARG, "d must be in [3, 65536]");
  if (bits < 1 || bits > 8) return fail(TQ_E_ARG, "bits must be in [1, 8]");
  if (!centroids || !boundaries) return fail(TQ_E_ARG, "output pointer is NULL");
  try {
    codebook_build(d, bits, centroids, boundaries);
  } catch (const std::bad_alloc&) {
    return fail(TQ_E_ARG, "out of host memory");
  }
  return TQ_OK;
}

tq_status tq_rotation_build(int32_t d, uint64_t seed, double* pi) {
  if (d < 1 || d > 1024) return fail(TQ_E_ARG, "d must be in [1, 1024]");
  if (!pi) return fail(TQ_E_ARG, "output pointer is NULL");
  try {
    rotation_build(d, seed, pi);
  } catch (const std::bad_alloc&) {
    return fail(TQ_E_ARG, "out of host memory");
  }
  return TQ_OK;
}

tq_status tq_hadamard_rotation_build(int32_t d, uint64_t seed, double* pi) {
  if (d < 1 || d > 1024 || (d & (d - 1))) return fail(TQ_E_ARG, "d must be a power of two in [1, 1024]");
  if (!pi) return fail(TQ_E_ARG, "output pointer is NULL");
  try {
    hadamard_rotation_build(d, seed, pi);
  } catch (const std::bad_alloc&) {
    return fail(TQ_E_ARG, "out of host memory");
  }
  return TQ_OK;
}

tq_status tq_sketch_build(int32_t m, int32_t d, uint64_t seed, double* s) {
  if (m < 1 || m > 1024 || d < 1 || d > 1024) return fail(TQ_E_ARG, "m and d must be in [1, 1024]");
  if (!s) return fail(TQ_E_ARG, "output pointer is NULL");
  gaussian_fill(seed, s, static_cast<size_t>(m) * d);
  return TQ_OK;
}

size_t tq_tables_bytes(void) { return sizeof(tq::Tables); }

tq_status tq_tables_build(const tq_spec* spec, void* host_buf, size_t bytes) {
  tq::Spec sp;
  if (tq_status st = check_spec(spec, &sp); st != TQ_OK) return st;
  if (!host_buf) return fail(TQ_E_ARG, "host_buf is NULL");
  if (bytes < sizeof(tq::Tables)) return fail(TQ_E_ARG, "host_buf smaller than tq_tables_bytes()");
  if (!aligned(host_buf, 16)) return fail(TQ_E_ARG, "host_buf must be 16-byte aligned");
  try {
    std::vector<unsigned char> raw(sizeof(tq::Tables) + 256, 0);
    auto* t = reinterpret_cast<tq::Tables*>((reinterpret_cast<uintptr_t>(raw.data()) + 255) &
                                            ~static_cast<uintptr_t>(255));
    t->magic = tq::TABLES_MAGIC;
    t->version = TQ_FORMAT_VERSION;
    t->bits[0] = sp.bits_lo;
    t->bits[1] = sp.bits_hi;
    t->split = sp.bits_lo == sp.bits_hi ? 128u : 64u;
    t->qjl_m = sp.qjl_m;
    t->layout = sp.layout;
    for (int h = 0; h < 2; ++h) {
      const int b = t->bits[h], L = 1 << b;
      std::vector<double> c(L), bd(L - 1);
      codebook_build(tq::D, b, c.data(), bd.data());
      if (b == 8) {
        if (h == 1) break;  // uniform width: one codebook
        t->cen16_scale[0] = t->cen16_scale[1] = 1.0f;
        for (int j = 0; j < 256; ++j) {
          t->bnd8[j] = j < 255 ? static_cast<float>(bd[j]) : INFINITY;
          t->cen8[j] = static_cast<float>(c[j]);
          t->cen16_8[j] = to_half(c[j]);
        }
        if (!(bd[0] > -0.5 && bd[254] < 0.5) ||
            !cell_table_8(t->bnd8, 255, t->cell8))
          return fail(TQ_E_UNSUPPORTED, "8-bit codebook boundaries too close for the code cell table");
        break;
      }
      // (the scale depends on the width alone: computed once per width)
      static std::atomic<double> scale_of[9];
      double sc = scale_of[b].load(std::memory_order_relaxed);
      if (!(sc >= 1.0)) {
        sc = centroid_scale(c.data(), L);
        scale_of[b].store(sc, std::memory_order_relaxed);
      }
      t->cen16_scale[h] = static_cast<float>(sc);
      for (int j = 0; j < 16; ++j) {
        t->bnd[h][j] = j < L - 1 ? static_cast<float>(bd[j]) : INFINITY;
        t->cen[h][j] = j < L ? static_cast<float>(c[j]) : 0.0f;
        t->cen16[h][j] = j < L ? to_half(c[j] * sc) : 0;
      }
      if (!cell_table_u(t->bnd[h], L - 1, t->cell[h]))
        return fail(TQ_E_UNSUPPORTED, "codebook boundaries too close for the code cell table");
    }
    std::vector<double> m(tq::D * tq::D);
    if (spec->rotation != TQ_ROT_HAAR) hadamard_rotation_build(tq::D, spec->rot_seed, m.data());
    else rotation_build(tq::D, spec->rot_seed, m.data());
    for (int i = 0; i < tq::D; ++i)
      for (int k = 0; k < tq::D; ++k) t->pit[k * tq::D + i] = static_cast<float>(m[i * tq::D + k]);
    for (int i = 0; i < tq::D * tq::D; ++i) {
      const uint16_t b0 = to_bf16(m[i]);
      const uint16_t b1 = to_bf16(m[i] - from_bf16(b0));
      const uint16_t b2 = to_bf16(m[i] - from_bf16(b0) - from_bf16(b1));
      t->pi_b16[0][i] = b0;
      t->pi_b16[1][i] = b1;
      t->pi_b16[2][i] = b2;
    }
    for (int i = 0; i < tq::D * tq::D; ++i) {
      t->pi[i] = static_cast<float>(m[i]);
      const double v = m[i] * tq::PI_SCALE;
      const uint16_t hi = to_half(v);
      t->pi_hi[i] = hi;
      t->pi_lo[i] = to_half(v - from_half(hi));
    }
    for (int lay = 0; lay < 2; ++lay)
      for (int w = 0; w < 2; ++w)
        for (int tt = 0; tt < 2; ++tt)
          for (int ks = 0; ks < 8; ++ks)
            for (int lane = 0; lane < 64; ++lane)
              for (int e = 0; e < 8; ++e) {
                const int row = tq::frag_row(lay, w, tt, lane), col = 16 * ks + 8 * (lane >> 5) + e;
                const int dst = ((((w * 2 + tt) * 8 + ks) * 64 + lane) * 8) + e;
                t->pi_frag[lay][0][dst] = t->pi_hi[row * tq::D + col];
                t->pi_frag[lay][1][dst] = t->pi_lo[row * tq::D + col];
              }
    if (sp.qjl_m) {
      gaussian_fill(spec->qjl_seed, m.data(), static_cast<size_t>(tq::QJL_M) * tq::D);
      for (int i = 0; i < tq::QJL_M; ++i)
        for (int k = 0; k < tq::D; ++k) t->sit[k * tq::QJL_M + i] = static_cast<float>(m[i * tq::D + k]);
      for (int i = 0; i < tq::QJL_M * tq::D; ++i) {
        t->s[i] = static_cast<float>(m[i]);
        const uint16_t hi = to_half(m[i]);
        t->s_hi[i] = hi;
        t->s_lo[i] = to_half(m[i] - from_half(hi));
      }
    }
    std::memcpy(host_buf, t, sizeof(tq::Tables));
  } catch (const std::bad_alloc&) {
    return fail(TQ_E_ARG, "out of host memory");
  }
  return TQ_OK;
}

size_t tq_code_bytes(const tq_spec* spec) {
  tq::Spec sp;
  if (check_spec(spec, &sp) != TQ_OK) return 0;
  return static_cast<size_t>(sp.code_bytes);
}

size_t tq_cache_code_bytes(const tq_spec* spec, int64_t cap) {
  tq::Spec sp;
  if (check_spec(spec, &sp) != TQ_OK || cap < 0) return 0;
  int64_t pos = cap;
  if (sp.layout == TQ_LAYOUT_TILED) pos = (cap + tq::TILE - 1) / tq::TILE * tq::TILE;
  return static_cast<size_t>(pos) * sp.code_bytes;
}

size_t tq_ip_workspace_bytes(void) { return tq::ip_workspace_bytes(); }

tq_status tq_ip_scores(const tq_spec* spec, const void* tables, const tq_cache* db, int64_t n_streams,
                       int64_t n_tok, const float* q, int32_t nq, float* scores, int64_t ld, void* workspace,
                       size_t ws_bytes, void* stream) {
  tq::Spec sp;
  if (tq_status st = check_spec(spec, &sp); st != TQ_OK) return st;
  if (sp.layout != TQ_LAYOUT_RECORD) return fail(TQ_E_UNSUPPORTED, "search needs the record layout");
  if (sp.bits_lo == 8) return fail(TQ_E_UNSUPPORTED, "search takes codes of at most 4 bits");
  if (sp.norm16) return fail(TQ_E_UNSUPPORTED, "search takes fp32 norms");
  if (tq_status st = check_tables(tables, sp, "search"); st != TQ_OK) return st;
  if (!db) return fail(TQ_E_ARG, "db is NULL");
  if (n_streams < 0 || n_tok < 0) return fail(TQ_E_ARG, "negative n_streams or n_tok");
  if (nq < 1 || nq > TQ_IP_MAX_QUERIES) return fail(TQ_E_UNSUPPORTED, "nq must be in [1, 64]");
  if (n_tok > db->cap) return fail(TQ_E_ARG, "n_tok exceeds the cache capacity");
  if (n_tok > (int64_t{1} << 24)) return fail(TQ_E_UNSUPPORTED, "at most 2^24 positions per stream");
  if (n_streams > 65535) return fail(TQ_E_UNSUPPORTED, "at most 65535 streams per call");
  if (ld < n_streams * n_tok) return fail(TQ_E_ARG, "ld smaller than n_streams * n_tok");
  if (n_streams == 0 || n_tok == 0) return TQ_OK;
  if (!q || !scores || !db->codes || !db->norms) return fail(TQ_E_ARG, "q, scores and db arrays must be non-NULL");
  if (sp.qjl_m && (!db->qjl_signs || !db->qjl_rnorms)) return fail(TQ_E_ARG, "db QJL arrays are NULL");
  if (!aligned(q, 4) || !aligned(scores, 4) || !aligned(db->codes, 16) || !aligned(db->norms, 16))
    return fail(TQ_E_ARG, "q and scores must be 4-byte, codes and norms 16-byte aligned");
  if (sp.qjl_m && (!aligned(db->qjl_signs, 16) || !aligned(db->qjl_rnorms, 16)))
    return fail(TQ_E_ARG, "QJL arrays must be 16-byte aligned");
  if (!workspace || ws_bytes < tq::ip_workspace_bytes()) return fail(TQ_E_WORKSPACE, "workspace too small");
  if (!aligned(workspace, 16)) return fail(TQ_E_ARG, "workspace must be 16-byte aligned");
  const hipError_t e = tq::launch_ip_scores(sp, static_cast<const tq::Tables*>(tables), *db, n_streams, n_tok, q, nq,
                                            scores, ld, workspace, static_cast<hipStream_t>(stream));
  return hip_status(e, "tq_ip_scores launch");
}

}  // extern "C"

namespace {

// Checks shared by both quantize entry points (everything but the ranges).
tq_status check_quantize(const tq_spec* spec, const void* tables, int32_t dtype, const tq_cache* cache,
                         tq::Spec* sp) {
  if (tq_status st = check_spec(spec, sp); st != TQ_OK) return st;
  if (tq_status st = check_tables(tables, *sp, "quantize"); st != TQ_OK) return st;
  if (dtype != TQ_F32 && dtype != TQ_BF16) return fail(TQ_E_ARG, "dtype must be TQ_F32 or TQ_BF16");
  if (!cache) return fail(TQ_E_ARG, "cache is NULL");
  if (cache->cap < 0) return fail(TQ_E_ARG, "negative cache cap");
  if (sp->layout == TQ_LAYOUT_TILED && cache->cap % tq::TILE)
    return fail(TQ_E_ARG, "tiled cache cap must be a multiple of 32");
  return TQ_OK;
}

tq_status check_quantize_arrays(const tq::Spec& sp, int32_t dtype, const void* x, int64_t x_stream_stride,
                                int64_t x_row_stride, int64_t max_tok, const tq_cache* cache) {
  const int64_t es = dtype == TQ_F32 ? 4 : 2;
  if (!x || !cache->codes || !cache->norms) return fail(TQ_E_ARG, "x, codes and norms must be non-NULL");
  if (!aligned(x, 16)) return fail(TQ_E_ARG, "x must be 16-byte aligned");
  if ((x_row_stride * es) % 16 || (x_stream_stride * es) % 16)
    return fail(TQ_E_ARG, "x strides must be multiples of 16 bytes");
  if (x_row_stride < tq::D && max_tok > 1) return fail(TQ_E_ARG, "x_row_stride smaller than d");
  if (!aligned(cache->codes, 16) || !aligned(cache->norms, 4))
    return fail(TQ_E_ARG, "codes must be 16-byte and norms 4-byte aligned");
  // 8-bit codes run only in the register-resident kernel (32-bit offsets)
  if (sp.bits_lo == 8 && (32 * x_row_stride * es >= (int64_t{1} << 30) || cache->cap >= (int64_t{1} << 31) - 64))
    return fail(TQ_E_UNSUPPORTED, "8-bit codes: x_row_stride * 32 rows must stay below 2^30 bytes and cap below 2^31 - 64");
  if (sp.qjl_m) {
    if (!cache->qjl_signs || !cache->qjl_rnorms) return fail(TQ_E_ARG, "QJL arrays must be non-NULL");
    if (!aligned(cache->qjl_signs, 16) || !aligned(cache->qjl_rnorms, 4))
      return fail(TQ_E_ARG, "qjl_signs must be 16-byte and qjl_rnorms 4-byte aligned");
  }
  return TQ_OK;
}

}  // namespace

extern "C" {

tq_status tq_quantize_kv(const tq_spec* spec, const void* tables, int32_t dtype, const void* x,
                         int64_t n_streams, int64_t n_tok, int64_t x_stream_stride,
                         int64_t x_row_stride, int64_t tok0, const tq_cache* cache, void* stream) {
  tq::Spec sp;
  if (tq_status st = check_quantize(spec, tables, dtype, cache, &sp); st != TQ_OK) return st;
  if (n_streams < 0 || n_tok < 0 || tok0 < 0) return fail(TQ_E_ARG, "negative size or offset");
  if (tok0 + n_tok > cache->cap) return fail(TQ_E_ARG, "tok0 + n_tok exceeds cache cap");
  if (n_streams == 0 || n_tok == 0) return TQ_OK;
  if (tq_status st = check_quantize_arrays(sp, dtype, x, x_stream_stride, x_row_stride, n_tok, cache); st != TQ_OK)
    return st;
  const tq::QSeq one{0, tok0, n_tok, 0, 0};
  const hipError_t e = tq::launch_quantize(sp, static_cast<const tq::Tables*>(tables), dtype, x, &one, 1, n_streams,
                                           x_stream_stride, x_row_stride, *cache, tq::PageMap{},
                                           static_cast<hipStream_t>(stream));
  return hip_status(e, "tq_quantize_kv launch");
}

tq_status tq_quantize_kv_ragged(const tq_spec* spec, const void* tables, int32_t dtype, const void* x,
                                int32_t batch, int32_t hkv, const int64_t* x_off, const int64_t* tok0,
                                const int64_t* n_tok, int64_t x_stream_stride, int64_t x_row_stride,
                                const tq_cache* cache, void* stream) {
  tq::Spec sp;
  if (tq_status st = check_quantize(spec, tables, dtype, cache, &sp); st != TQ_OK) return st;
  if (batch < 0 || hkv <= 0) return fail(TQ_E_ARG, "batch must be >= 0 and hkv > 0");
  if (batch == 0) return TQ_OK;
  if (!x_off || !tok0 || !n_tok) return fail(TQ_E_ARG, "x_off, tok0 and n_tok must be non-NULL");
  const int64_t es = dtype == TQ_F32 ? 4 : 2;
  std::vector<tq::QSeq> seqs;
  seqs.reserve(static_cast<size_t>(batch));
  int64_t max_tok = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (n_tok[b] < 0 || tok0[b] < 0 || x_off[b] < 0) return fail(TQ_E_ARG, "negative size or offset");
    if (tok0[b] + n_tok[b] > cache->cap) return fail(TQ_E_ARG, "tok0 + n_tok exceeds cache cap");
    if ((x_off[b] * es) % 16) return fail(TQ_E_ARG, "x offsets must be multiples of 16 bytes");
    if (n_tok[b] == 0) continue;
    max_tok = std::max(max_tok, n_tok[b]);
    seqs.push_back(tq::QSeq{x_off[b], tok0[b], n_tok[b], static_cast<int64_t>(b) * hkv, 0});
  }
  if (seqs.empty()) return TQ_OK;
  if (tq_status st = check_quantize_arrays(sp, dtype, x, x_stream_stride, x_row_stride, max_tok, cache); st != TQ_OK)
    return st;
  const hipError_t e = tq::launch_quantize(sp, static_cast<const tq::Tables*>(tables), dtype, x, seqs.data(),
                                           static_cast<int64_t>(seqs.size()), hkv, x_stream_stride, x_row_stride,
                                           *cache, tq::PageMap{}, static_cast<hipStream_t>(stream));
  return hip_status(e, "tq_quantize_kv_ragged launch");
}

size_t tq_attend_workspace_bytes(const tq_attn* attn) {
  if (!attn || attn->batch < 0 || attn->hq <= 0 || attn->hkv <= 0 || attn->max_len < 0) return 0;
  return tq::plan_attend(*attn).ws_bytes;
}

}  // extern "C"

namespace tq {

tq_status set_error(tq_status st, const char* msg) { return fail(st, msg); }

// Every decode entry point: the contiguous caches (block_table == NULL) and
// the paged pools, with a caller's workspace or the static scratch.
tq_status attend_checked(const tq_spec* ks, const void* ktables, const tq_cache* kc, const tq_spec* vs,
                         const void* vtables, const tq_cache* vc, const tq_attn* attn, const float* q,
                         const uint16_t* sink_k, const uint16_t* sink_v, const int32_t* seq_lens,
                         const int32_t* block_table, int32_t max_pages, int64_t n_pages, float* out,
                         void* workspace, size_t ws_bytes, void* stream, const char* what) {
  tq::Spec ksp, vsp;
  if (tq_status st = check_spec(ks, &ksp); st != TQ_OK) return st;
  if (tq_status st = check_spec(vs, &vsp); st != TQ_OK) return st;
  if (ksp.layout != TQ_LAYOUT_RECORD) return fail(TQ_E_UNSUPPORTED, "keys must use the record layout");
  if (vsp.layout != TQ_LAYOUT_TILED) return fail(TQ_E_UNSUPPORTED, "values must use the tiled layout");
  if (vsp.qjl_m) return fail(TQ_E_UNSUPPORTED, "values carry no QJL sketch");
  if (vsp.bits_lo == 8) return fail(TQ_E_UNSUPPORTED, "8-bit codes are for keys (record layout)");
  if (ksp.bits_lo == 8 && !(vsp.bits_lo == vsp.bits_hi && (vsp.bits_lo == 2 || vsp.bits_lo == 3)))
    return fail(TQ_E_UNSUPPORTED, "8-bit keys decode with values of 2 or 3 bits (uniform)");
  if (ksp.norm16 != vsp.norm16) return fail(TQ_E_UNSUPPORTED, "K and V specs must agree on norm_f16");
  if (tq_status st = check_tables(ktables, ksp, "key"); st != TQ_OK) return st;
  if (tq_status st = check_tables(vtables, vsp, "value"); st != TQ_OK) return st;
  if (!attn || !kc || !vc) return fail(TQ_E_ARG, "attn, kc and vc must be non-NULL");
  const tq_attn& a = *attn;
  if (a.batch < 0 || a.hq <= 0 || a.hkv <= 0) return fail(TQ_E_ARG, "batch, hq, hkv out of range");
  if (a.hq % a.hkv) return fail(TQ_E_ARG, "hq must be a multiple of hkv");
  if (a.hq / a.hkv > 16) return fail(TQ_E_UNSUPPORTED, "at most 16 query heads per KV head");
  if (a.batch > 65535) return fail(TQ_E_UNSUPPORTED, "at most 65535 sequences per call");
  if (a.sink < 0 || a.max_len < 0) return fail(TQ_E_ARG, "negative sink or max_len");
  if (a.sink > 512) return fail(TQ_E_UNSUPPORTED, "at most 512 sink tokens");
  if (!(a.v_skip >= 0.0f) || !(a.v_skip < 1.0f)) return fail(TQ_E_ARG, "v_skip must be in [0, 1)");
  if (!std::isfinite(a.scale)) return fail(TQ_E_ARG, "scale must be finite");
  if (a.batch == 0) return TQ_OK;
  if (block_table) {
    if (kc->cap != TQ_PAGE_TOKENS || vc->cap != TQ_PAGE_TOKENS)
      return fail(TQ_E_ARG, "page pools must have cap == TQ_PAGE_TOKENS");
    if (max_pages < 1 || n_pages < 1 || n_pages > (int64_t{1} << 30))
      return fail(TQ_E_ARG, "max_pages and n_pages must be positive (n_pages <= 2^30)");
    if (a.max_len - a.sink > static_cast<int64_t>(max_pages) * TQ_PAGE_TOKENS)
      return fail(TQ_E_ARG, "max_len - sink exceeds max_pages pages");
    if (a.max_len - a.sink > (int64_t{1} << 24)) return fail(TQ_E_UNSUPPORTED, "at most 2^24 compressed tokens");
    if (!aligned(block_table, 4)) return fail(TQ_E_ARG, "block_table must be 4-byte aligned");
  } else {
    if (vc->cap % tq::TILE || kc->cap % tq::TILE) return fail(TQ_E_ARG, "cache caps must be multiples of 32");
    if (vc->cap > (int64_t{1} << 24) || kc->cap > (int64_t{1} << 24))
      return fail(TQ_E_UNSUPPORTED, "cache caps above 2^24 positions");
    if (a.max_len - a.sink > std::min(kc->cap, vc->cap))
      return fail(TQ_E_ARG, "max_len - sink exceeds the cache capacity");
  }
  if (!q || !out || !seq_lens) return fail(TQ_E_ARG, "q, out and seq_lens must be non-NULL");
  if (!kc->codes || !kc->norms || !vc->codes || !vc->norms) return fail(TQ_E_ARG, "cache arrays are NULL");
  if (ksp.qjl_m && (!kc->qjl_signs || !kc->qjl_rnorms)) return fail(TQ_E_ARG, "key QJL arrays are NULL");
  if (a.sink > 0 && (!sink_k || !sink_v)) return fail(TQ_E_ARG, "sink_k and sink_v are required when sink > 0");
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(kc->codes, 16) || !aligned(vc->codes, 16) ||
      !aligned(kc->norms, 16) || !aligned(vc->norms, 16) || !aligned(seq_lens, 4))
    return fail(TQ_E_ARG, "q, out, codes and norms must be 16-byte aligned");
  if (a.sink > 0 && (!aligned(sink_k, 16) || !aligned(sink_v, 16)))
    return fail(TQ_E_ARG, "sink arrays must be 16-byte aligned");
  if (ksp.qjl_m && (!aligned(kc->qjl_signs, 16) || !aligned(kc->qjl_rnorms, 16)))
    return fail(TQ_E_ARG, "QJL arrays must be 16-byte aligned");
  const tq::AttendPlan plan = tq::plan_attend(a);
  if (!workspace || ws_bytes < plan.ws_bytes) return fail(TQ_E_WORKSPACE, "workspace too small");
  if (!aligned(workspace, 16)) return fail(TQ_E_ARG, "workspace must be 16-byte aligned");
  const hipError_t e = tq::launch_attend(ksp, static_cast<const tq::Tables*>(ktables), *kc, vsp,
                                         static_cast<const tq::Tables*>(vtables), *vc, a, plan, q,
                                         sink_k, sink_v, seq_lens, out, workspace,
                                         static_cast<hipStream_t>(stream), block_table, max_pages,
                                         static_cast<int>(n_pages));
  return hip_status(e, what);
}

}  // namespace tq

extern "C" {

tq_status tq_attend_decode(const tq_spec* ks, const void* ktables, const tq_cache* kc,
                           const tq_spec* vs, const void* vtables, const tq_cache* vc,
                           const tq_attn* attn, const float* q, const uint16_t* sink_k,
                           const uint16_t* sink_v, const int32_t* seq_lens, float* out,
                           void* workspace, size_t ws_bytes, void* stream) {
  return tq::attend_checked(ks, ktables, kc, vs, vtables, vc, attn, q, sink_k, sink_v, seq_lens, nullptr, 0, 0,
                            out, workspace, ws_bytes, stream, "tq_attend_decode launch");
}

tq_status tq_attend_decode_paged(const tq_spec* ks, const void* ktables, const tq_cache* kpool,
                                 const tq_spec* vs, const void* vtables, const tq_cache* vpool,
                                 const tq_attn* attn, const float* q, const uint16_t* sink_k,
                                 const uint16_t* sink_v, const int32_t* seq_lens, const int32_t* block_table,
                                 int32_t max_pages, int64_t n_pages, float* out, void* workspace,
                                 size_t ws_bytes, void* stream) {
  if (!block_table) return fail(TQ_E_ARG, "block_table is NULL");
  return tq::attend_checked(ks, ktables, kpool, vs, vtables, vpool, attn, q, sink_k, sink_v, seq_lens, block_table,
                            max_pages, n_pages, out, workspace, ws_bytes, stream, "tq_attend_decode_paged launch");
}

tq_status tq_quantize_kv_paged(const tq_spec* spec, const void* tables, int32_t dtype, const void* x,
                               int32_t batch, int32_t hkv, const int64_t* x_off, const int64_t* pos0,
                               const int64_t* n_tok, int64_t x_stream_stride, int64_t x_row_stride,
                               const int32_t* block_table, int32_t max_pages, int64_t n_pages,
                               const tq_cache* pool, void* stream) {
  tq::Spec sp;
  if (tq_status st = check_quantize(spec, tables, dtype, pool, &sp); st != TQ_OK) return st;
  if (pool->cap != TQ_PAGE_TOKENS) return fail(TQ_E_ARG, "the page pool must have cap == TQ_PAGE_TOKENS");
  if (batch < 0 || hkv <= 0 || max_pages < 1 || n_pages < 1 || n_pages > (int64_t{1} << 30))
    return fail(TQ_E_ARG, "batch >= 0, hkv > 0, max_pages > 0 and 0 < n_pages <= 2^30 required");
  if (batch == 0) return TQ_OK;
  if (!x_off || !pos0 || !n_tok) return fail(TQ_E_ARG, "x_off, pos0 and n_tok must be non-NULL");
  if (!block_table || !aligned(block_table, 4)) return fail(TQ_E_ARG, "block_table must be non-NULL and 4-byte aligned");
  const int64_t es = dtype == TQ_F32 ? 4 : 2;
  std::vector<tq::QSeq> seqs;
  int64_t max_tok = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (n_tok[b] < 0 || pos0[b] < 0 || x_off[b] < 0) return fail(TQ_E_ARG, "negative size or offset");
    if ((x_off[b] * es) % 16) return fail(TQ_E_ARG, "x offsets must be multiples of 16 bytes");
    if (pos0[b] + n_tok[b] > static_cast<int64_t>(max_pages) * TQ_PAGE_TOKENS)
      return fail(TQ_E_ARG, "pos0 + n_tok exceeds max_pages pages");
    if (n_tok[b] == 0) continue;
    max_tok = std::max(max_tok, n_tok[b]);
    seqs.push_back(tq::QSeq{x_off[b], pos0[b], n_tok[b], 0, b});
  }
  if (seqs.empty()) return TQ_OK;
  if (tq_status st = check_quantize_arrays(sp, dtype, x, x_stream_stride, x_row_stride, max_tok, pool); st != TQ_OK)
    return st;
  const tq::PageMap pm{block_table, max_pages, n_pages};
  const hipError_t e = tq::launch_quantize(sp, static_cast<const tq::Tables*>(tables), dtype, x, seqs.data(),
                                           static_cast<int64_t>(seqs.size()), hkv, x_stream_stride, x_row_stride,
                                           *pool, pm, static_cast<hipStream_t>(stream));
  return hip_status(e, "tq_quantize_kv_paged launch");
}

}  // extern "C"
