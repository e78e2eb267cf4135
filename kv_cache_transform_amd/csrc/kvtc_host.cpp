// Host core of libkvtc: codec state, calibration (page "KV Cache Transform
// Coding for Compact Storage in LLM Inference", section 2A), artifact and
// stream sizes, device-state upload, job validation and kernel launches.
#include <zlib.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <memory>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "kvtc_internal.h"
#include "kvtc_linalg.h"

using namespace kvtc;

namespace {

thread_local std::string g_err;

kvtc_status fail(kvtc_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

struct Slot {
  bool calibrated = false;
  std::vector<uint8_t> widths;   // [F/G]; with cwidths, each group's largest component width
  std::vector<uint8_t> cwidths;  // [F] a width per component, or empty (a width per group)
  std::vector<float> mu32;       // [F]
  std::vector<double> lam;       // [F]
  std::vector<float> V32;        // [F][r_eff]
  int n_act = 0, r_eff = 0, record_bytes = 0;
  bool fold = false;             // the encode folds the mean into the product (see folds_mean)
  uint64_t slot_id = 0;
  std::vector<uint8_t> bytes;    // serialized slot (including the id)
};

uint64_t fnv1a64(const uint8_t* p, size_t n) {
  uint64_t h = 0xCBF29CE484222325ull;
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 0x100000001B3ull;
  }
  return h;
}

template <class T>
void put(std::vector<uint8_t>& b, const T& v) {
  const uint8_t* p = reinterpret_cast<const uint8_t*>(&v);
  b.insert(b.end(), p, p + sizeof(T));
}

uint16_t f32_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

float bf16_to_f32(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// fp32 -> fp16 bits, round to nearest even, with subnormals.
uint16_t f32_to_f16(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) return (uint16_t)(sign | (ax > 0x7F800000u ? 0x7E00u : 0x7C00u));
  if (ax >= 0x47800000u) return (uint16_t)(sign | 0x7C00u);  // >= 65536
  if (ax < 0x38800000u) {                                    // below 2^-14
    float a;
    std::memcpy(&a, &ax, 4);
    const uint32_t m = (uint32_t)std::nearbyint(a * 16777216.0f);  // units of 2^-24
    return (uint16_t)(sign | m);
  }
  const uint32_t mant = ax & 0x7FFFFFu;
  uint32_t h = ((((ax >> 23) - 112u)) << 10) | (mant >> 13);
  const uint32_t rem = mant & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;
  return (uint16_t)(sign | h);
}

}  // namespace

struct kvtc_codec {
  kvtc_params p;
  int F = 0, n_g = 0;
  std::vector<Slot> slots;                // n_layers * 2
  std::mutex mu;                          // guards the version counters
  uint64_t calib_version = 0;
  uint64_t uploaded_version = ~0ull;
  const uint8_t* d_state = nullptr;
  size_t d_state_bytes = 0;
  const int32_t* d_zero = nullptr;        // a zero word in the device state
};

namespace {

kvtc_status check_params(const kvtc_params* p) {
  if (!p) return fail(KVTC_E_INVALID, "null params");
  if (p->n_layers <= 0 || p->kv_heads <= 0 || p->head_dim <= 0)
    return fail(KVTC_E_INVALID, "n_layers, kv_heads and head_dim must be positive");
  const long F = (long)p->kv_heads * p->head_dim;
  if (F > 65536) return fail(KVTC_E_INVALID, "F too large");
  if (p->group <= 0 || p->group % 8 || F % p->group)
    return fail(KVTC_E_INVALID, "group must be a positive multiple of 8 dividing F");
  if (F / p->group > 512) return fail(KVTC_E_INVALID, "more than 512 groups");
  if (p->max_bits < 0 || p->max_bits > 8) return fail(KVTC_E_INVALID, "max_bits must be in 0..8");
  if (!(p->bits_per_value >= 0.f) || !std::isfinite(p->bits_per_value))
    return fail(KVTC_E_INVALID, "bits_per_value must be finite and >= 0");
  if (p->sink < 0 || p->window < 0) return fail(KVTC_E_INVALID, "negative sink or window");
  if (p->dtype != KVTC_F32 && p->dtype != KVTC_BF16) return fail(KVTC_E_INVALID, "bad dtype");
  return KVTC_OK;
}

long budget_bits(const kvtc_params& p) {
  return (long)std::floor((double)p.bits_per_value * (double)(p.kv_heads * p.head_dim));
}

int group_cost(int b, int G) { return G * b + (b > 0 ? kScaleBits : 0); }

// DP bit allocation (section 2A): minimise sum_g D[g][b_g] subject to
// sum_g cost(b_g) <= budget. f[g][u] is the least distortion of groups g..
// spending exactly u bits, f[g][u] = min_b D[g][b] + f[g+1][u - cost(b)],
// evaluated from the last group so that every objective is the nested sum
// D[0] + (D[1] + (... + 0)). Ties: fewest bits, then the lexicographically
// largest widths (largest b first when walking forward).
std::vector<uint8_t> dp_allocate(const std::vector<double>& D, int n_g, int nb, int G, long budget) {
  const double INF = std::numeric_limits<double>::infinity();
  const long U = budget + 1;
  std::vector<double> f((size_t)(n_g + 1) * U, INF);
  f[(size_t)n_g * U + 0] = 0.0;
  for (int g = n_g - 1; g >= 0; --g) {
    const double* nxt = f.data() + (size_t)(g + 1) * U;
    double* cur = f.data() + (size_t)g * U;
    for (long u = 0; u < U; ++u) {
      double best = INF;
      for (int b = 0; b < nb; ++b) {
        const long c = group_cost(b, G);
        if (c <= u && nxt[u - c] < INF) {
          const double v = D[(size_t)g * nb + b] + nxt[u - c];
          if (v < best) best = v;
        }
      }
      cur[u] = best;
    }
  }
  long u = 0;
  for (long v = 1; v < U; ++v)
    if (f[v] < f[u]) u = v;
  std::vector<uint8_t> w(n_g, 0);
  for (int g = 0; g < n_g; ++g) {
    for (int b = nb - 1; b >= 0; --b) {
      const long c = group_cost(b, G);
      if (c <= u && D[(size_t)g * nb + b] + f[(size_t)(g + 1) * U + u - c] == f[(size_t)g * U + u]) {
        w[g] = (uint8_t)b;
        u -= c;
        break;
      }
    }
  }
  return w;
}

// Bytes of a group's code chunk with a width per component: the widths'
// sum rounded up to whole bytes.
int chunk_bytes_pc(const uint8_t* cw, int G) {
  int sum = 0;
  for (int i = 0; i < G; ++i) sum += cw[i];
  return (sum + 7) / 8;
}

void finish_slot(const kvtc_params& p, int layer, int kind, Slot& s) {
  const int F = p.kv_heads * p.head_dim, G = p.group, n_g = F / G;
  const bool pc = !s.cwidths.empty();
  s.n_act = 0;
  int code_bytes = 0;
  for (int g = 0; g < n_g; ++g)
    if (s.widths[g]) {
      ++s.n_act;
      code_bytes += pc ? chunk_bytes_pc(s.cwidths.data() + (size_t)g * G, G) : G * s.widths[g] / 8;
    }
  s.r_eff = s.n_act * G;
  s.record_bytes = 8 * s.n_act + code_bytes;
  // Whether the encode folds the mean into the product (bf16 input only):
  // c = V'^T x - V'^T mu32 with the token multiplied as stored (an exact bf16
  // operand, one MFMA term), instead of centring each token first (two
  // terms). The fp32 rounding error of the folded product scales with |x|
  // rather than |x - mu|; when the calibration's mean is no larger than its
  // spread (|mu32|^2 <= sum of the covariance eigenvalues = E|x - mu|^2) |x|
  // is within a factor of about sqrt(2) of |x - mu|, and so is the error.
  // KVTC_ENCODE_CENTRED=1 in the environment when the slot is finished keeps
  // it on the centred product (for comparisons).
  {
    double m2 = 0.0, tr = 0.0;
    for (float v : s.mu32) m2 += (double)v * v;
    for (double v : s.lam) tr += v;
    const char* env = std::getenv("KVTC_ENCODE_CENTRED");
    const bool centred = env && env[0] == '1';
    s.fold = p.dtype == KVTC_BF16 && s.r_eff > 0 && m2 <= tr && !centred;
  }
  std::vector<uint8_t> b;
  b.insert(b.end(), {'K', 'V', 'T', 'S'});
  const int32_t hdr[7] = {layer, kind, F, G, s.n_act, s.r_eff, pc ? 1 : 0};
  for (int32_t v : hdr) put(b, v);
  const std::vector<uint8_t>& wv = pc ? s.cwidths : s.widths;
  const size_t nw = wv.size(), wpad = (nw + 7) / 8 * 8;
  for (size_t i = 0; i < wpad; ++i) b.push_back(i < nw ? wv[i] : 0);
  for (float v : s.mu32) put(b, v);
  for (double v : s.lam) put(b, v);
  for (float v : s.V32) put(b, v);
  s.slot_id = fnv1a64(b.data(), b.size());
  put(b, s.slot_id);
  s.bytes.swap(b);
  s.calibrated = true;
}

// Global allocation over several tensors sharing one budget: minimise the
// sum of their distortions subject to sum of their bits <= n * budget and at
// most max_active active groups per tensor. Costs are multiples of
// unit = gcd(G, 64) bits, so the tables run in units. Per tensor,
// f[g][u][r] = least distortion of groups g.. spending exactly u units with
// at most r active groups (the per-tensor recurrence with a count of active
// groups); e_s[u] = f_s[0][u][cap]; H[s][U] = min_u e_s[u] + H[s+1][U - u].
// Ties: fewest total bits, then the most bits to the tensor earliest in the
// list, then the per-tensor rule (largest b first).
struct CapTable {
  int n_g, top, cap;
  std::vector<double> f;
  double& at(int g, long u, int r) { return f[((size_t)g * (top + 1) + u) * (cap + 1) + r]; }
};

void cap_table(const std::vector<double>& D, int n_g, int nb, int G, int unit, int top, int cap,
               CapTable& t) {
  const double INF = std::numeric_limits<double>::infinity();
  t.n_g = n_g;
  t.top = top;
  t.cap = cap;
  t.f.assign((size_t)(n_g + 1) * (top + 1) * (cap + 1), INF);
  for (int r = 0; r <= cap; ++r) t.at(n_g, 0, r) = 0.0;
  for (int g = n_g - 1; g >= 0; --g)
    for (int r = 0; r <= cap; ++r)
      for (long u = 0; u <= top; ++u) {
        double best = INF;
        for (int b = 0; b < nb; ++b) {
          const long c = group_cost(b, G) / unit;
          const int rr = r - (b > 0 ? 1 : 0);
          if (rr < 0 || c > u) continue;
          const double v = D[(size_t)g * nb + b] + t.at(g + 1, u - c, rr);
          if (v < best) best = v;
        }
        t.at(g, u, r) = best;
      }
}

std::vector<std::vector<uint8_t>> dp_allocate_global(const std::vector<std::vector<double>>& Ds, int n_g,
                                                     int nb, int G, long budget, int max_active) {
  const double INF = std::numeric_limits<double>::infinity();
  const int S = (int)Ds.size();
  int unit = kScaleBits;
  while (G % unit) unit /= 2;                  // gcd(G, 64); G is a multiple of 8
  const long Bu = (long)S * budget / unit;
  const int cap = std::min(max_active, n_g);
  const int top = (int)std::min<long>(Bu, (long)cap * group_cost(nb - 1, G) / unit);
  std::vector<std::vector<double>> e(S);
  CapTable t;
  for (int s = 0; s < S; ++s) {
    cap_table(Ds[s], n_g, nb, G, unit, top, cap, t);
    e[s].resize(top + 1);
    for (int u = 0; u <= top; ++u) e[s][u] = t.at(0, u, cap);
  }
  std::vector<double> H((size_t)(S + 1) * (Bu + 1), INF);
  auto h = [&](int s, long U) -> double& { return H[(size_t)s * (Bu + 1) + U]; };
  h(S, 0) = 0.0;
  for (int s = S - 1; s >= 0; --s)
    for (int u = 0; u <= top; ++u) {
      if (!(e[s][u] < INF)) continue;
      for (long U = u; U <= Bu; ++U) {
        const double v = e[s][u] + h(s + 1, U - u);
        if (v < h(s, U)) h(s, U) = v;
      }
    }
  long U = 0;
  for (long v = 1; v <= Bu; ++v)
    if (h(0, v) < h(0, U)) U = v;
  std::vector<std::vector<uint8_t>> out(S, std::vector<uint8_t>(n_g, 0));
  for (int s = 0; s < S; ++s) {
    long u = std::min<long>(U, top);
    for (; u >= 0; --u)
      if (e[s][u] < INF && e[s][u] + h(s + 1, U - u) == h(s, U)) break;
    if (u < 0) u = 0;                          // unreachable: H[s][U] came from some u
    U -= u;
    cap_table(Ds[s], n_g, nb, G, unit, top, cap, t);
    int r = cap;
    for (int g = 0; g < n_g; ++g)
      for (int b = nb - 1; b >= 0; --b) {
        const long c = group_cost(b, G) / unit;
        const int rr = r - (b > 0 ? 1 : 0);
        if (c <= u && rr >= 0 && Ds[s][(size_t)g * nb + b] + t.at(g + 1, u - c, rr) == t.at(g, u, r)) {
          out[s][g] = (uint8_t)b;
          u -= c;
          r = rr;
          break;
        }
      }
  }
  return out;
}

// The DP widths with at most KVTC_MAX_REFF / G active groups (the kernels'
// limit): dp_allocate's, or, when they need more, the allocation minimising
// the distortion under both the budget and the cap (dp_allocate_global of
// the one tensor, which equals dp_allocate whenever the cap does not bind).
std::vector<uint8_t> dp_allocate_capped(const std::vector<double>& D, int n_g, int nb, int G, long budget) {
  std::vector<uint8_t> w = dp_allocate(D, n_g, nb, G, budget);
  int n_act = 0;
  for (uint8_t b : w) n_act += b ? 1 : 0;
  if (n_act * G <= KVTC_MAX_REFF) return w;
  return dp_allocate_global({D}, n_g, nb, G, budget, KVTC_MAX_REFF / G)[0];
}

// Rows [s, n - w) of one calibration tensor in fp64, centred on their mean.
struct CalRows {
  long n_r = 0;
  std::vector<double> X;    // [n_r][F], centred
  std::vector<double> mu;   // [F]
};

kvtc_status load_centred(const kvtc_params& p, int F, const void* host_kv, int64_t n_tokens, int threads,
                         CalRows& r) {
  const long n_r = (long)n_tokens - p.sink - p.window;
  if (n_tokens < 0 || n_r < 1) return fail(KVTC_E_INVALID, "need at least one row after sink and window");
  r.n_r = n_r;
  r.X.assign((size_t)n_r * F, 0.0);
  parallel_for((int)std::min<long>(n_r, 1L << 30), threads, [&](int t) {
    const size_t src_row = (size_t)(t + p.sink) * F;
    double* xr = r.X.data() + (size_t)t * F;
    if (p.dtype == KVTC_BF16) {
      const uint16_t* s = (const uint16_t*)host_kv + src_row;
      for (int f = 0; f < F; ++f) xr[f] = bf16_to_f32(s[f]);
    } else {
      const float* s = (const float*)host_kv + src_row;
      for (int f = 0; f < F; ++f) xr[f] = s[f];
    }
  });
  // Mean (section 2B subtracts it before the transform).
  r.mu.assign(F, 0.0);
  for (long t = 0; t < n_r; ++t) {
    const double* xr = r.X.data() + (size_t)t * F;
    for (int f = 0; f < F; ++f) r.mu[f] += xr[f];
  }
  for (int f = 0; f < F; ++f) r.mu[f] /= (double)n_r;
  parallel_for((int)n_r, threads, [&](int t) {
    double* xr = r.X.data() + (size_t)t * F;
    for (int f = 0; f < F; ++f) xr[f] -= r.mu[f];
  });
  return KVTC_OK;
}

// cov += X^T X (upper triangle computed, then mirrored) of centred rows.
void add_scatter(const CalRows& r, int F, int threads, std::vector<double>& cov) {
  std::vector<double> sc((size_t)F * F);
  gemm_f64(F, F, (int)r.n_r, r.X.data(), 1, F, r.X.data(), F, sc.data(), F, true, threads);
  for (int i = 0; i < F; ++i)
    for (int j = 0; j < i; ++j) sc[(size_t)i * F + j] = sc[(size_t)j * F + i];
  for (size_t k = 0; k < sc.size(); ++k) cov[k] += sc[k];
}

// Eigenvectors of the scatter / n_rows: the right singular vectors of the
// centred rows (the SVD of section 2A), eigenvalues sigma^2 / n, sorted by
// descending eigenvalue (stable), largest-magnitude entry of each made
// positive. V[f][j], column j = component j.
kvtc_status eigen_basis(int F, std::vector<double>& cov, double n_rows, std::vector<double>& V,
                        std::vector<double>& lam) {
  for (auto& v : cov) v /= n_rows;
  std::vector<double> evals, zt;
  if (sym_eigen(F, cov, evals, zt) != 0) return fail(KVTC_E_INVALID, "eigensolver did not converge");
  std::vector<int> order(F);
  for (int j = 0; j < F; ++j) order[j] = j;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return evals[a] > evals[b]; });
  V.assign((size_t)F * F, 0.0);
  lam.assign(F, 0.0);
  for (int j = 0; j < F; ++j) {
    const double* z = zt.data() + (size_t)order[j] * F;
    lam[j] = evals[order[j]];
    int imax = 0;
    for (int f = 1; f < F; ++f)
      if (std::fabs(z[f]) > std::fabs(z[imax])) imax = f;
    const double sgn = z[imax] < 0 ? -1.0 : 1.0;
    for (int f = 0; f < F; ++f) V[(size_t)f * F + j] = sgn * z[f];
  }
  return KVTC_OK;
}

// Empirical distortion table D[g][b] of the quantizer on the calibration
// coefficients C = X V (fp64).
std::vector<double> distortion(const CalRows& r, int F, int G, int nb, const std::vector<double>& V,
                               int threads) {
  const long n_r = r.n_r;
  const int n_g = F / G;
  std::vector<double> C((size_t)n_r * F);
  gemm_f64((int)n_r, F, F, r.X.data(), F, 1, V.data(), F, C.data(), F, false, threads);
  std::vector<double> D((size_t)n_g * nb, 0.0);
  parallel_for(n_g, threads, [&](int g) {
    std::vector<double> acc(nb, 0.0);
    for (long t = 0; t < n_r; ++t) {
      const double* cg = C.data() + (size_t)t * F + (size_t)g * G;
      double mn = cg[0], mx = cg[0], e0 = 0.0;
      for (int i = 0; i < G; ++i) {
        mn = std::min(mn, cg[i]);
        mx = std::max(mx, cg[i]);
        e0 += cg[i] * cg[i];
      }
      acc[0] += e0;
      const double scale = mx - mn;
      for (int b = 1; b < nb; ++b) {
        if (!(scale > 0)) continue;  // every value equals the shift: no error
        const double k = (double)((1 << b) - 1);
        const double inv = k / scale, step = scale / k;
        double e = 0.0;
        for (int i = 0; i < G; ++i) {
          double q = std::nearbyint((cg[i] - mn) * inv);
          q = std::min(std::max(q, 0.0), k);
          const double d = cg[i] - (mn + q * step);
          e += d * d;
        }
        acc[b] += e;
      }
    }
    for (int b = 0; b < nb; ++b) D[(size_t)g * nb + b] = acc[b] / (double)n_r;
  });
  return D;
}

// Per-component distortion Dc[j][b] (a width per component): component j
// on b levels of its group's grid (the min and range of all G components),
// b = 0 its energy.
std::vector<double> distortion_pc(const CalRows& r, int F, int G, int nb, const std::vector<double>& V,
                                  int threads) {
  const long n_r = r.n_r;
  const int n_g = F / G;
  std::vector<double> C((size_t)n_r * F);
  gemm_f64((int)n_r, F, F, r.X.data(), F, 1, V.data(), F, C.data(), F, false, threads);
  std::vector<double> D((size_t)F * nb, 0.0);
  parallel_for(n_g, threads, [&](int g) {
    std::vector<double> acc((size_t)G * nb, 0.0);
    for (long t = 0; t < n_r; ++t) {
      const double* cg = C.data() + (size_t)t * F + (size_t)g * G;
      double mn = cg[0], mx = cg[0];
      for (int i = 1; i < G; ++i) {
        mn = std::min(mn, cg[i]);
        mx = std::max(mx, cg[i]);
      }
      const double scale = mx - mn;
      for (int i = 0; i < G; ++i) {
        acc[(size_t)i * nb] += cg[i] * cg[i];
        if (!(scale > 0)) continue;  // every value equals the shift: no error
        for (int b = 1; b < nb; ++b) {
          const double k = (double)((1 << b) - 1);
          double q = std::nearbyint((cg[i] - mn) * (k / scale));
          q = std::min(std::max(q, 0.0), k);
          const double d = cg[i] - (mn + q * (scale / k));
          acc[(size_t)i * nb + b] += d * d;
        }
      }
    }
    for (int i = 0; i < G; ++i)
      for (int b = 0; b < nb; ++b) D[((size_t)g * G + i) * nb + b] = acc[(size_t)i * nb + b] / (double)n_r;
  });
  return D;
}

int group_cost_pc(int sum) { return sum == 0 ? 0 : kScaleBits + 8 * ((sum + 7) / 8); }

// Widths per component minimising sum_j Dc[j][b_j] within the budget, a
// group costing 64 + 8 ceil(sum_j b_j / 8) bits when any b_j > 0. Per group,
// e[i][s] = least distortion of components i.. of the group with widths
// summing to s (nested from the last component); across groups,
// f[g][u] = min_s e_g[0][s] + f[g+1][u - cost(s)] (nested from the last
// group). Ties: fewest bits, then the largest s for the earliest group,
// then the largest widths first inside a group.
// Per-component allocation (a width per component, cost 64 + 8 ceil(sum/8)
// bits per active group). PcInner: per group g, e(g, i, s) = least
// distortion of components i.. of the group whose widths sum to s.
struct PcInner {
  int n_g, G, nb, smax;
  std::vector<double> E;
  double& e(int g, int i, int sm) { return E[((size_t)g * (G + 1) + i) * (smax + 1) + sm]; }
};
PcInner pc_inner(const std::vector<double>& Dc, int F, int nb, int G) {
  const double INF = std::numeric_limits<double>::infinity();
  PcInner P{F / G, G, nb, (nb - 1) * G, {}};
  P.E.assign((size_t)P.n_g * (G + 1) * (P.smax + 1), INF);
  for (int g = 0; g < P.n_g; ++g) {
    const double* D = Dc.data() + (size_t)g * G * nb;
    P.e(g, G, 0) = 0.0;
    for (int i = G - 1; i >= 0; --i)
      for (int sm = 0; sm <= P.smax; ++sm) {
        double best = INF;
        for (int b = 0; b < nb && b <= sm; ++b) {
          const double nx = P.e(g, i + 1, sm - b);
          if (nx < INF) {
            const double v = D[(size_t)i * nb + b] + nx;
            if (v < best) best = v;
          }
        }
        P.e(g, i, sm) = best;
      }
  }
  return P;
}
// Group g's component widths summing to sm, largest width first.
void pc_components(PcInner& P, const std::vector<double>& Dc, int g, int sm, std::vector<uint8_t>& w) {
  const double INF = std::numeric_limits<double>::infinity();
  const int G = P.G, nb = P.nb;
  const double* D = Dc.data() + (size_t)g * G * nb;
  for (int i = 0; i < G; ++i)
    for (int b = std::min(nb - 1, sm); b >= 0; --b) {
      const double nx = P.e(g, i + 1, sm - b);
      if (nx < INF && D[(size_t)i * nb + b] + nx == P.e(g, i, sm)) {
        w[(size_t)g * G + i] = (uint8_t)b;
        sm -= b;
        break;
      }
    }
}

// At most R active groups: f(g, u, r) = least distortion of groups g.. at
// exactly u bits with at most r of them active; the same tie order as the
// plain allocation (fewest bits, largest sum for the earliest group, largest
// widths first).
std::vector<uint8_t> dp_allocate_pc_capped(PcInner& P, const std::vector<double>& Dc, long budget, int R) {
  const double INF = std::numeric_limits<double>::infinity();
  const int n_g = P.n_g, smax = P.smax;
  const long U = budget + 1;
  std::vector<double> f((size_t)(n_g + 1) * U * (R + 1), INF);
  auto F_ = [&](int g, long u, int r) -> double& { return f[((size_t)g * U + u) * (R + 1) + r]; };
  for (int r = 0; r <= R; ++r) F_(n_g, 0, r) = 0.0;
  for (int g = n_g - 1; g >= 0; --g)
    for (long u = 0; u < U; ++u)
      for (int r = 0; r <= R; ++r) {
        double best = INF;
        for (int sm = 0; sm <= smax; ++sm) {
          const long c = group_cost_pc(sm);
          const int rr = r - (sm > 0 ? 1 : 0);
          if (c > u || rr < 0 || !(P.e(g, 0, sm) < INF)) continue;
          const double nx = F_(g + 1, u - c, rr);
          if (nx < INF) {
            const double v = P.e(g, 0, sm) + nx;
            if (v < best) best = v;
          }
        }
        F_(g, u, r) = best;
      }
  long u = 0;
  for (long v = 1; v < U; ++v)
    if (F_(0, v, R) < F_(0, u, R)) u = v;
  std::vector<uint8_t> w((size_t)n_g * P.G, 0);
  int r = R;
  for (int g = 0; g < n_g; ++g) {
    int sm = smax;
    for (; sm > 0; --sm) {
      const long c = group_cost_pc(sm);
      if (c <= u && r >= 1 && P.e(g, 0, sm) < INF &&
          P.e(g, 0, sm) + F_(g + 1, u - c, r - 1) == F_(g, u, r))
        break;
    }
    u -= group_cost_pc(sm);   // sm == 0: the group stays inactive
    if (sm > 0) --r;
    pc_components(P, Dc, g, sm, w);
  }
  return w;
}

// The plain allocation: f(g, u) = min_s E_g(s) + f(g + 1, u - cost(s)); with
// max_active, the capped one whenever the plain result has more active
// groups than that (reading Q3c).
std::vector<uint8_t> dp_allocate_pc(const std::vector<double>& Dc, int F, int nb, int G, long budget,
                                    int max_active) {
  const double INF = std::numeric_limits<double>::infinity();
  PcInner P = pc_inner(Dc, F, nb, G);
  const int n_g = P.n_g, smax = P.smax;
  const long U = budget + 1;
  std::vector<double> f((size_t)(n_g + 1) * U, INF);
  f[(size_t)n_g * U] = 0.0;
  for (int g = n_g - 1; g >= 0; --g)
    for (long u = 0; u < U; ++u) {
      double best = INF;
      for (int sm = 0; sm <= smax; ++sm) {
        const long c = group_cost_pc(sm);
        if (c > u || !(P.e(g, 0, sm) < INF)) continue;
        const double nx = f[(size_t)(g + 1) * U + u - c];
        if (nx < INF) {
          const double v = P.e(g, 0, sm) + nx;
          if (v < best) best = v;
        }
      }
      f[(size_t)g * U + u] = best;
    }
  long u = 0;
  for (long v = 1; v < U; ++v)
    if (f[v] < f[u]) u = v;
  std::vector<uint8_t> w(F, 0);
  int n_act = 0;
  for (int g = 0; g < n_g; ++g) {
    int sm = smax;
    for (; sm >= 0; --sm) {
      const long c = group_cost_pc(sm);
      if (c <= u && P.e(g, 0, sm) < INF && P.e(g, 0, sm) + f[(size_t)(g + 1) * U + u - c] == f[(size_t)g * U + u])
        break;
    }
    if (sm < 0) sm = 0;   // unreachable: f[g][u] came from some s
    u -= group_cost_pc(sm);
    if (sm > 0) ++n_act;
    pc_components(P, Dc, g, sm, w);
  }
  if (n_act > max_active) return dp_allocate_pc_capped(P, Dc, budget, max_active);
  return w;
}

std::vector<float> to_f32(const std::vector<double>& v) { return std::vector<float>(v.begin(), v.end()); }

// A calibrated slot from its widths, mean, eigenvalues and full basis
// (V[f][j] in fp32, F x F): the active groups' columns in component order.
kvtc_status build_slot(const kvtc_params& p, int layer, int kind, const std::vector<uint8_t>& widths,
                       const std::vector<double>& mu, const std::vector<double>& lam,
                       const std::vector<float>& V, Slot& s,
                       const std::vector<uint8_t>& cwidths = std::vector<uint8_t>()) {
  const int F = p.kv_heads * p.head_dim, G = p.group, n_g = F / G;
  int n_act = 0;
  for (int g = 0; g < n_g; ++g) n_act += widths[g] ? 1 : 0;
  if (n_act * G > KVTC_MAX_REFF)
    return fail(KVTC_E_UNSUPPORTED, "allocation needs more than KVTC_MAX_REFF active components");
  s = Slot();
  s.widths = widths;
  s.mu32.resize(F);
  for (int f = 0; f < F; ++f) s.mu32[f] = (float)mu[f];
  s.lam = lam;
  s.V32.resize((size_t)F * n_act * G);
  int a = 0;
  for (int g = 0; g < n_g; ++g) {
    if (!widths[g]) continue;
    for (int i = 0; i < G; ++i)
      for (int f = 0; f < F; ++f) s.V32[(size_t)f * n_act * G + a * G + i] = V[(size_t)f * F + g * G + i];
    ++a;
  }
  s.cwidths = cwidths;
  finish_slot(p, layer, kind, s);
  return KVTC_OK;
}

bool slot_index(const kvtc_codec* c, int layer, int kind, int* idx) {
  if (!c || layer < 0 || layer >= c->p.n_layers || (kind != KVTC_K && kind != KVTC_V)) return false;
  *idx = layer * 2 + kind;
  return true;
}

void split_rows(long T, const kvtc_params& p, uint32_t* s1, uint32_t* w1, uint32_t* tc) {
  const long s = std::min<long>(p.sink, T);
  const long w = std::min<long>(p.window, T - s);
  *s1 = (uint32_t)s;
  *w1 = (uint32_t)w;
  *tc = (uint32_t)(T - s - w);
}

size_t elem_bytes(int dtype) { return dtype == KVTC_F32 ? 4 : 2; }

size_t stream_bytes(const kvtc_codec* c, const Slot& s, long T) {
  uint32_t s1, w1, tc;
  split_rows(T, c->p, &s1, &w1, &tc);
  return kHeaderBytes + (size_t)(s1 + w1) * c->F * elem_bytes(c->p.dtype) + (size_t)tc * s.record_bytes;
}

// Whether the encode folds the mean into the product for this slot (decided
// when the slot is finished, see finish_slot).
bool folds_mean(const kvtc_codec*, const Slot& s) { return s.calibrated && s.fold; }

// Decode staging of one job: stg_block_bytes(ks) per block of kDecTok
// compressed tokens.
size_t job_staging_bytes(const Slot& s, uint32_t tc) {
  const int ks = (int)(align_up((size_t)s.r_eff, 16) / 16);
  return align_up((size_t)((tc + kDecTok - 1) / kDecTok) * stg_block_bytes(ks), kAlign);
}

// Byte offset of the workspace sink behind the status words of n jobs.
size_t sink_offset(int32_t n) { return align_up((size_t)std::max(n, 1) * sizeof(uint64_t), kAlign); }

}  // namespace

extern "C" {

const char* kvtc_version(void) { return "kvtc 0.1 gfx950"; }

const char* kvtc_last_error(void) { return g_err.c_str(); }

kvtc_status kvtc_create(const kvtc_params* params, kvtc_codec** out) {
  if (!out) return fail(KVTC_E_INVALID, "null output pointer");
  *out = nullptr;
  const kvtc_status st = check_params(params);
  if (st != KVTC_OK) return st;
  auto c = std::make_unique<kvtc_codec>();
  c->p = *params;
  c->F = params->kv_heads * params->head_dim;
  c->n_g = c->F / params->group;
  c->slots.resize((size_t)params->n_layers * 2);
  *out = c.release();
  return KVTC_OK;
}

void kvtc_destroy(kvtc_codec* codec) { delete codec; }

kvtc_status kvtc_calibrate(kvtc_codec* c, int32_t layer, int32_t kind, const void* host_kv,
                           int64_t n_tokens, int32_t threads) {
  int idx;
  if (!slot_index(c, layer, kind, &idx)) return fail(KVTC_E_INVALID, "bad codec, layer or kind");
  if (!host_kv) return fail(KVTC_E_INVALID, "null calibration data");
  if (threads <= 0) threads = std::max(1u, std::thread::hardware_concurrency());
  const kvtc_params& p = c->p;
  const int F = c->F, nb = p.max_bits + 1;
  CalRows r;
  kvtc_status st = load_centred(p, F, host_kv, n_tokens, threads, r);
  if (st != KVTC_OK) return st;
  std::vector<double> cov((size_t)F * F, 0.0), V, lam;
  add_scatter(r, F, threads, cov);
  st = eigen_basis(F, cov, (double)r.n_r, V, lam);
  if (st != KVTC_OK) return st;
  const std::vector<double> D = distortion(r, F, p.group, nb, V, threads);
  Slot s;
  st = build_slot(p, layer, kind, dp_allocate_capped(D, c->n_g, nb, p.group, budget_bits(p)), r.mu, lam,
                  to_f32(V), s);
  if (st != KVTC_OK) return st;
  c->slots[idx] = std::move(s);
  std::lock_guard<std::mutex> lk(c->mu);
  ++c->calib_version;
  return KVTC_OK;
}

kvtc_status kvtc_calibrate_set(kvtc_codec* c, const kvtc_calib_input* in, int32_t n, uint32_t flags,
                               int32_t threads) {
  if (!c || !in || n < 1) return fail(KVTC_E_INVALID, "bad codec or inputs");
  if (flags & ~(uint32_t)(KVTC_CAL_SHARED_BASIS | KVTC_CAL_GLOBAL_BUDGET | KVTC_CAL_COMPONENT_WIDTHS))
    return fail(KVTC_E_INVALID, "unknown calibration flags");
  const bool pcw = (flags & KVTC_CAL_COMPONENT_WIDTHS) != 0;
  if (pcw && (flags & KVTC_CAL_GLOBAL_BUDGET))
    return fail(KVTC_E_INVALID, "component widths take a budget per tensor");
  if (threads <= 0) threads = std::max(1u, std::thread::hardware_concurrency());
  const kvtc_params& p = c->p;
  const int F = c->F, G = p.group, n_g = c->n_g, nb = p.max_bits + 1;
  // Tensors in (layer, kind) order; each at most once.
  std::vector<int> ord(n);
  for (int i = 0; i < n; ++i) {
    int idx;
    if (!slot_index(c, in[i].layer, in[i].kind, &idx)) return fail(KVTC_E_INVALID, "bad layer or kind");
    if (!in[i].host_kv) return fail(KVTC_E_INVALID, "null calibration data");
    if (in[i].n_tokens - p.sink - p.window < 1)
      return fail(KVTC_E_INVALID, "need at least one row after sink and window");
    ord[i] = i;
  }
  auto key = [&](int i) { return in[i].layer * 2 + in[i].kind; };
  std::sort(ord.begin(), ord.end(), [&](int a, int b) { return key(a) < key(b); });
  for (int i = 1; i < n; ++i)
    if (key(ord[i]) == key(ord[i - 1])) return fail(KVTC_E_INVALID, "a (layer, kind) appears twice");

  // Means, bases and distortion tables.
  std::vector<std::vector<double>> mus(n), lams(n), Ds(n);
  std::vector<std::vector<float>> Vs(n);        // per tensor, or per kind when shared
  std::vector<int> vref(n);                     // which entry of Vs / lams a tensor uses
  if (flags & KVTC_CAL_SHARED_BASIS) {
    for (int kind = 0; kind < 2; ++kind) {
      std::vector<int> same;
      for (int i : ord)
        if (in[i].kind == kind) same.push_back(i);
      if (same.empty()) continue;
      // one basis over the pooled rows, each tensor centred on its own mean
      std::vector<double> cov((size_t)F * F, 0.0), V, lam;
      double n_rows = 0;
      for (int i : same) {
        CalRows r;
        kvtc_status st = load_centred(p, F, in[i].host_kv, in[i].n_tokens, threads, r);
        if (st != KVTC_OK) return st;
        add_scatter(r, F, threads, cov);
        n_rows += (double)r.n_r;
        mus[i] = std::move(r.mu);
      }
      kvtc_status st = eigen_basis(F, cov, n_rows, V, lam);
      if (st != KVTC_OK) return st;
      for (int i : same) {
        CalRows r;
        st = load_centred(p, F, in[i].host_kv, in[i].n_tokens, threads, r);
        if (st != KVTC_OK) return st;
        Ds[i] = pcw ? distortion_pc(r, F, G, nb, V, threads) : distortion(r, F, G, nb, V, threads);
        vref[i] = same[0];
      }
      Vs[same[0]] = to_f32(V);
      lams[same[0]] = std::move(lam);
    }
  } else {
    for (int i : ord) {
      CalRows r;
      kvtc_status st = load_centred(p, F, in[i].host_kv, in[i].n_tokens, threads, r);
      if (st != KVTC_OK) return st;
      std::vector<double> cov((size_t)F * F, 0.0), V, lam;
      add_scatter(r, F, threads, cov);
      st = eigen_basis(F, cov, (double)r.n_r, V, lam);
      if (st != KVTC_OK) return st;
      Ds[i] = pcw ? distortion_pc(r, F, G, nb, V, threads) : distortion(r, F, G, nb, V, threads);
      mus[i] = std::move(r.mu);
      Vs[i] = to_f32(V);
      lams[i] = std::move(lam);
      vref[i] = i;
    }
  }

  // Widths: one DP per tensor, or one over the whole set.
  std::vector<std::vector<uint8_t>> widths(n);
  if (flags & KVTC_CAL_GLOBAL_BUDGET) {
    std::vector<std::vector<double>> ds;
    for (int i : ord) ds.push_back(Ds[i]);
    const auto ws = dp_allocate_global(ds, n_g, nb, G, budget_bits(p), KVTC_MAX_REFF / G);
    for (int k = 0; k < n; ++k) widths[ord[k]] = ws[k];
  } else if (pcw) {
    for (int i : ord) widths[i] = dp_allocate_pc(Ds[i], F, nb, G, budget_bits(p), KVTC_MAX_REFF / G);
  } else {
    for (int i : ord) widths[i] = dp_allocate_capped(Ds[i], n_g, nb, G, budget_bits(p));
  }

  // Build every slot first, so a failure leaves the codec unchanged.
  std::vector<Slot> out(n);
  for (int i : ord) {
    std::vector<uint8_t> gw = widths[i], cw;
    if (pcw) {   // a group's width: its largest component's (nonzero: active)
      cw.swap(gw);
      gw.assign(n_g, 0);
      for (int g = 0; g < n_g; ++g)
        for (int k = 0; k < G; ++k) gw[g] = std::max(gw[g], cw[(size_t)g * G + k]);
    }
    kvtc_status st = build_slot(p, in[i].layer, in[i].kind, gw, mus[i], lams[vref[i]], Vs[vref[i]],
                                out[i], cw);
    if (st != KVTC_OK) return st;
  }
  for (int i : ord) c->slots[key(i)] = std::move(out[i]);
  std::lock_guard<std::mutex> lk(c->mu);
  ++c->calib_version;
  return KVTC_OK;
}

kvtc_status kvtc_slot_info_get(const kvtc_codec* c, int32_t layer, int32_t kind, kvtc_slot_info* info) {
  int idx;
  if (!slot_index(c, layer, kind, &idx) || !info) return fail(KVTC_E_INVALID, "bad arguments");
  std::memset(info, 0, sizeof(*info));
  const Slot& s = c->slots[idx];
  info->calibrated = s.calibrated;
  if (!s.calibrated) return KVTC_OK;
  info->n_act = s.n_act;
  info->r_eff = s.r_eff;
  info->record_bytes = s.record_bytes;
  info->slot_id = s.slot_id;
  info->per_component = s.cwidths.empty() ? 0 : 1;
  info->folded_mean = folds_mean(c, s) ? 1 : 0;
  for (int g = 0; g < c->n_g && g < 512; ++g) info->widths[g] = s.widths[g];
  return KVTC_OK;
}

kvtc_status kvtc_save(const kvtc_codec* c, void* buf, size_t cap, size_t* written) {
  if (!c || !written) return fail(KVTC_E_INVALID, "bad arguments");
  std::vector<uint8_t> b;
  b.insert(b.end(), {'K', 'V', 'T', 'A'});
  put(b, (uint32_t)kFormatVersion);
  const int32_t hdr[7] = {c->p.n_layers, c->p.kv_heads, c->p.head_dim, c->p.sink,
                          c->p.window, c->p.group, c->p.max_bits};
  for (int32_t v : hdr) put(b, v);
  put(b, c->p.bits_per_value);
  put(b, (int32_t)c->p.dtype);
  int32_t n = 0;
  for (const Slot& s : c->slots) n += s.calibrated;
  put(b, n);
  for (const Slot& s : c->slots)
    if (s.calibrated) b.insert(b.end(), s.bytes.begin(), s.bytes.end());
  *written = b.size();
  if (!buf) return KVTC_OK;
  if (cap < b.size()) return fail(KVTC_E_CAPACITY, "artifact buffer too small");
  std::memcpy(buf, b.data(), b.size());
  return KVTC_OK;
}

kvtc_status kvtc_load(const void* buf, size_t n, kvtc_codec** out) {
  if (!buf || !out) return fail(KVTC_E_INVALID, "bad arguments");
  *out = nullptr;
  const uint8_t* b = (const uint8_t*)buf;
  size_t off = 0;
  auto need = [&](size_t k) { return off + k <= n; };
  auto rd32 = [&](int32_t* v) {
    std::memcpy(v, b + off, 4);
    off += 4;
  };
  if (!need(48) || std::memcmp(b, "KVTA", 4) != 0) return fail(KVTC_E_CORRUPT, "bad artifact magic");
  off = 4;
  int32_t ver;
  rd32(&ver);
  if (ver != kFormatVersion) return fail(KVTC_E_CORRUPT, "bad artifact version");
  kvtc_params p;
  rd32(&p.n_layers);
  rd32(&p.kv_heads);
  rd32(&p.head_dim);
  rd32(&p.sink);
  rd32(&p.window);
  rd32(&p.group);
  rd32(&p.max_bits);
  std::memcpy(&p.bits_per_value, b + off, 4);
  off += 4;
  rd32(&p.dtype);
  int32_t n_slots;
  rd32(&n_slots);
  kvtc_codec* c = nullptr;
  kvtc_status st = kvtc_create(&p, &c);
  if (st != KVTC_OK) return fail(KVTC_E_CORRUPT, std::string("artifact parameters: ") + g_err);
  std::unique_ptr<kvtc_codec> guard(c);
  const int F = c->F, G = p.group, n_g = c->n_g;
  for (int i = 0; i < n_slots; ++i) {
    const size_t start = off;
    if (!need(32) || std::memcmp(b + off, "KVTS", 4) != 0) return fail(KVTC_E_CORRUPT, "bad slot magic");
    off += 4;
    int32_t layer, kind, sF, sG, n_act, r_eff, mode;
    rd32(&layer);
    rd32(&kind);
    rd32(&sF);
    rd32(&sG);
    rd32(&n_act);
    rd32(&r_eff);
    rd32(&mode);
    int idx;
    if (!slot_index(c, layer, kind, &idx) || sF != F || sG != G || r_eff != n_act * G ||
        n_act < 0 || n_act > n_g || (mode != 0 && mode != 1))
      return fail(KVTC_E_CORRUPT, "inconsistent slot header");
    if (r_eff > KVTC_MAX_REFF) return fail(KVTC_E_UNSUPPORTED, "slot exceeds KVTC_MAX_REFF");
    const size_t nw = mode ? (size_t)F : (size_t)n_g, wpad = (nw + 7) / 8 * 8;
    const size_t body = wpad + 4 * (size_t)F + 8 * (size_t)F + 4 * (size_t)F * r_eff + 8;
    if (!need(body)) return fail(KVTC_E_CORRUPT, "truncated slot");
    Slot s;
    if (mode) {
      s.cwidths.assign(b + off, b + off + F);
      s.widths.assign(n_g, 0);
      for (int g = 0; g < n_g; ++g)
        for (int i = 0; i < G; ++i) s.widths[g] = std::max(s.widths[g], s.cwidths[(size_t)g * G + i]);
    } else {
      s.widths.assign(b + off, b + off + n_g);
    }
    off += wpad;
    int cnt = 0;
    for (uint8_t w : s.widths) {
      if (w > p.max_bits) return fail(KVTC_E_CORRUPT, "width above max_bits");
      cnt += w ? 1 : 0;
    }
    if (cnt != n_act) return fail(KVTC_E_CORRUPT, "n_act does not match widths");
    s.mu32.resize(F);
    std::memcpy(s.mu32.data(), b + off, 4 * (size_t)F);
    off += 4 * (size_t)F;
    s.lam.resize(F);
    std::memcpy(s.lam.data(), b + off, 8 * (size_t)F);
    off += 8 * (size_t)F;
    s.V32.resize((size_t)F * r_eff);
    std::memcpy(s.V32.data(), b + off, 4 * (size_t)F * r_eff);
    off += 4 * (size_t)F * r_eff;
    uint64_t id;
    std::memcpy(&id, b + off, 8);
    if (fnv1a64(b + start, off - start) != id) return fail(KVTC_E_CORRUPT, "slot id mismatch");
    off += 8;
    finish_slot(p, layer, kind, s);
    c->slots[idx] = std::move(s);
  }
  c->calib_version = 1;
  *out = guard.release();
  return KVTC_OK;
}

size_t kvtc_device_state_bytes(const kvtc_codec* c) {
  if (!c) return 0;
  size_t n = align_up(c->slots.size() * sizeof(DevSlot), kAlign) + kAlign;   // table, zero block
  for (const Slot& s : c->slots) {
    if (!s.calibrated) continue;
    const size_t r_enc = align_up((size_t)s.r_eff, 32), r_dec = align_up((size_t)s.r_eff, 16);
    n += 2 * align_up(4 * (size_t)c->F, kAlign) + align_up(2 * r_enc * c->F, kAlign) +
         align_up(2 * (size_t)c->F * r_dec, kAlign) + align_up(4 * r_enc, kAlign);
    if (!s.cwidths.empty()) n += align_up(4 * (size_t)s.r_eff, kAlign);
  }
  return n;
}

kvtc_status kvtc_upload(kvtc_codec* c, void* d_state, size_t bytes, hipStream_t stream) {
  if (!c || !d_state) return fail(KVTC_E_INVALID, "bad arguments");
  if ((uintptr_t)d_state % kAlign) return fail(KVTC_E_INVALID, "device state must be 256-byte aligned");
  const size_t need = kvtc_device_state_bytes(c);
  if (bytes < need) return fail(KVTC_E_CAPACITY, "device state buffer too small");
  if (c->p.group != 16 && c->p.group != 32)
    return fail(KVTC_E_UNSUPPORTED, "the kernels support group sizes 16 and 32");
  if (c->F % 64) return fail(KVTC_E_UNSUPPORTED, "the kernels need F to be a multiple of 64");
  std::vector<uint8_t> h(need, 0);
  std::vector<DevSlot> table(c->slots.size());
  std::memset(table.data(), 0, table.size() * sizeof(DevSlot));
  const size_t zero_off = align_up(c->slots.size() * sizeof(DevSlot), kAlign);
  size_t off = zero_off + kAlign;
  const int F = c->F, G = c->p.group;
  for (size_t i = 0; i < c->slots.size(); ++i) {
    const Slot& s = c->slots[i];
    DevSlot& d = table[i];
    if (!s.calibrated) continue;
    const int r = s.r_eff;
    const int r_enc = (int)align_up(r, 32), r_dec = (int)align_up(r, 16);
    d.calibrated = 1;
    d.n_act = s.n_act;
    d.r_eff = r;
    d.record_bytes = s.record_bytes;
    d.r_enc = r_enc;
    d.r_dec = r_dec;
    d.G = G;
    d.F = F;
    d.slot_id = s.slot_id;
    const bool pc = !s.cwidths.empty();
    d.pc = pc ? 1 : 0;
    const bool fold = folds_mean(c, s);
    d.fold = fold ? 1 : 0;
    int a = 0, chunk = 8 * s.n_act;
    for (int g = 0; g < c->n_g; ++g) {
      if (!s.widths[g]) continue;
      d.width[a] = s.widths[g];
      d.chunk_off[a] = (uint16_t)chunk;
      chunk += pc ? chunk_bytes_pc(s.cwidths.data() + (size_t)g * G, G) : G * s.widths[g] / 8;
      ++a;
    }
    d.mu_off = off;
    std::memcpy(h.data() + off, s.mu32.data(), 4 * (size_t)F);
    off += align_up(4 * (size_t)F, kAlign);
    d.venc_off = off;
    uint16_t* venc = (uint16_t*)(h.data() + off);  // V'^T [r_enc][F] bf16
    for (int j = 0; j < r; ++j)
      for (int f = 0; f < F; ++f) venc[(size_t)j * F + f] = f32_to_bf16(s.V32[(size_t)f * r + j]);
    off += align_up(2 * (size_t)r_enc * F, kAlign);
    d.vdec_off = off;
    // V' (F x r_dec, fp16, zero past r_eff) in the order the decode loads
    // its MFMA A operands: for feature block b (32 features) and K step k (16
    // components), 64 lanes x 8 values, lane 32 h + t holding
    // V'[32 b + t][16 k + 8 h + i], i = 0..7; one wave's operand is 1 KB of
    // contiguous memory.
    uint16_t* vdec = (uint16_t*)(h.data() + off);
    const int nks = r_dec / 16;
    for (int f = 0; f < F; ++f)
      for (int j = 0; j < r; ++j) {
        const size_t lane = 32 * (size_t)((j % 16) / 8) + (size_t)(f % 32);
        const size_t frag = (size_t)(f / 32) * nks + (size_t)(j / 16);
        vdec[(frag * 64 + lane) * 8 + (size_t)(j % 8)] =
            f32_to_f16(bf16_to_f32(f32_to_bf16(s.V32[(size_t)f * r + j])));
      }
    off += align_up(2 * (size_t)F * r_dec, kAlign);
    // Centring (section 2B subtracts the mean before the transform). The
    // encode subtracts mu_hi = bf16_rne(mu32) from each token in fp32 (exact
    // for bf16 tokens whenever token and mean lie within a factor 2^8 of each
    // other, so the error scales with |x - mu| and not with |x|) and starts
    // its accumulators at -V'^T (mu32 - mu_hi), this small remainder's
    // projection in fp64 rounded once. A slot that folds the mean (see
    // folds_mean) multiplies the raw token and starts at -V'^T mu32.
    d.mhi_off = off;
    float* mhi = (float*)(h.data() + off);
    for (int f = 0; f < F; ++f) mhi[f] = bf16_to_f32(f32_to_bf16(s.mu32[f]));
    off += align_up(4 * (size_t)F, kAlign);
    d.cmu_off = off;
    float* cmu = (float*)(h.data() + off);
    for (int j = 0; j < r; ++j) {
      double acc = 0.0;
      for (int f = 0; f < F; ++f)
        acc += ((double)s.mu32[f] - (fold ? 0.0 : (double)mhi[f])) *
               (double)bf16_to_f32(f32_to_bf16(s.V32[(size_t)f * r + j]));
      cmu[j] = (float)acc;
    }
    off += align_up(4 * (size_t)r_enc, kAlign);
    if (pc) {
      // per active component: (bit position in the record << 8) | width
      d.pcw_off = off;
      uint32_t* pcw = (uint32_t*)(h.data() + off);
      int aa = 0;
      for (int g = 0; g < c->n_g; ++g) {
        if (!s.widths[g]) continue;
        uint32_t bit = 8u * d.chunk_off[aa];
        for (int i = 0; i < G; ++i) {
          const uint32_t w = s.cwidths[(size_t)g * G + i];
          pcw[aa * G + i] = (bit << 8) | w;
          bit += w;
        }
        ++aa;
      }
      off += align_up(4 * (size_t)r, kAlign);
    }
  }
  std::memcpy(h.data(), table.data(), table.size() * sizeof(DevSlot));
  hipError_t e = hipMemcpyAsync(d_state, h.data(), need, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(KVTC_E_HIP, std::string("upload: ") + hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(c->mu);
  c->d_state = (const uint8_t*)d_state;
  c->d_state_bytes = need;
  c->d_zero = (const int32_t*)((const uint8_t*)d_state + zero_off);
  c->uploaded_version = c->calib_version;
  return KVTC_OK;
}

size_t kvtc_encoded_bytes(const kvtc_codec* c, int32_t layer, int32_t kind, int64_t n_tokens) {
  int idx;
  if (!slot_index(c, layer, kind, &idx) || n_tokens < 0 || !c->slots[idx].calibrated) return 0;
  return stream_bytes(c, c->slots[idx], n_tokens);
}

size_t kvtc_workspace_bytes(int32_t max_jobs) { return sink_offset(max_jobs) + kSinkBytes; }

size_t kvtc_staging_bytes(const kvtc_codec* c, const kvtc_job* jobs, int32_t n_jobs) {
  if (!c || !jobs || n_jobs <= 0) return 0;
  size_t n = 0;
  for (int i = 0; i < n_jobs; ++i) {
    int idx;
    if (!slot_index(c, jobs[i].layer, jobs[i].kind, &idx) || !c->slots[idx].calibrated) return 0;
    uint32_t s1, w1, tc;
    split_rows(jobs[i].n_tokens, c->p, &s1, &w1, &tc);
    n += job_staging_bytes(c->slots[idx], tc);
  }
  return n;
}

size_t kvtc_decode_workspace_bytes(const kvtc_codec* c, const kvtc_job* jobs, int32_t n_jobs) {
  // 0 flags jobs the codec cannot decode; otherwise the status words and the
  // sink, then the staging of the two-stage schedule.
  if (!c || !jobs || n_jobs <= 0) return 0;
  for (int i = 0; i < n_jobs; ++i) {
    int idx;
    if (!slot_index(c, jobs[i].layer, jobs[i].kind, &idx) || !c->slots[idx].calibrated) return 0;
  }
  return kvtc_workspace_bytes(n_jobs) + kvtc_staging_bytes(c, jobs, n_jobs);
}

}  // extern "C"

namespace {

enum class Mode { Encode, Unpack, Restore, Decode, Pack, UnpackCodes };

// Launch stamps for the workspace status words (0 is never issued).
uint32_t next_epoch() {
  static std::atomic<uint32_t> counter{0};
  uint32_t e = ++counter;
  if (e == 0) e = ++counter;
  return e;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Validate jobs [0, n) on the host and fill LaunchArgs batches. Jobs are
// grouped (stably) by the kernel shape they need (encode: r_enc / 32,
// decode and restore: r_dec / 16) and cut into batches of at most
// kMaxLaunchJobs; each job keeps its own status word (its index in `jobs`).
kvtc_status plan(kvtc_codec* c, Mode mode, const kvtc_job* jobs, int n, int out_dtype, void* d_ws,
                 uint8_t* d_staging, size_t staging_bytes, std::vector<LaunchArgs>& batches,
                 std::vector<int>& shape, std::vector<size_t>& lds) {
  if (!c || !jobs || n <= 0 || n > KVTC_MAX_JOBS) return fail(KVTC_E_INVALID, "bad codec, jobs or job count");
  if (!d_ws || !aligned16(d_ws)) return fail(KVTC_E_INVALID, "workspace must be non-null and aligned");
  const bool dec = mode == Mode::Unpack || mode == Mode::Restore || mode == Mode::Decode;
  if (dec && out_dtype != KVTC_F32 && out_dtype != KVTC_BF16) return fail(KVTC_E_INVALID, "bad output dtype");
  const int F = c->F;
  const size_t out_esz = elem_bytes(out_dtype);
  // Per-job validation and the fields that do not depend on the batch.
  std::vector<JobDesc> desc(n);
  std::vector<int> key(n), pcj(n, 0);   // pcj: launch class (decode: pc slots; encode: folded mean)
  std::vector<size_t> st_off(n, 0);
  size_t st_total = 0;
  for (int i = 0; i < n; ++i) {
    const kvtc_job& j = jobs[i];
    int idx;
    if (!slot_index(c, j.layer, j.kind, &idx)) return fail(KVTC_E_INVALID, "job: bad layer or kind");
    const Slot& s = c->slots[idx];
    if (!s.calibrated) return fail(KVTC_E_NOT_CALIBRATED, "job: (layer, kind) is not calibrated");
    if (j.n_tokens < 0 || j.n_tokens > (int64_t)INT32_MAX) return fail(KVTC_E_INVALID, "job: bad n_tokens");
    if (!j.dst || !aligned16(j.dst)) return fail(KVTC_E_INVALID, "job: dst must be non-null and 16-byte aligned");
    if (!j.src || !aligned16(j.src)) return fail(KVTC_E_INVALID, "job: src must be non-null and 16-byte aligned");
    // what the kernels read from src: the KV rows (encode, and the
    // passthrough rows of the pack hook) or the whole stream
    const bool reads_rows = mode == Mode::Encode || mode == Mode::Pack;
    const size_t src_need = reads_rows ? (size_t)j.n_tokens * F * elem_bytes(c->p.dtype) : stream_bytes(c, s, j.n_tokens);
    if (j.src_capacity < src_need)
      return fail(KVTC_E_CAPACITY, reads_rows ? "job: src_capacity below n_tokens rows" : "job: src_capacity below kvtc_encoded_bytes");
    JobDesc& d = desc[i];
    std::memset(&d, 0, sizeof(d));
    d.src = j.src;
    d.dst = j.dst;
    d.T = (uint32_t)j.n_tokens;
    split_rows(j.n_tokens, c->p, &d.s1, &d.w1, &d.tc);
    d.slot = idx;
    d.layer = j.layer;
    d.kind = j.kind;
    d.status_idx = i;
    d.bs_shift = -1;
    if (!s.cwidths.empty() && (mode == Mode::Pack || mode == Mode::UnpackCodes))
      return fail(KVTC_E_UNSUPPORTED, "the pack and unpack hooks take group widths");
    if (mode == Mode::Encode || mode == Mode::Pack) {
      if (j.dst_capacity < stream_bytes(c, s, j.n_tokens))
        return fail(KVTC_E_CAPACITY, "job: dst_capacity below kvtc_encoded_bytes");
      key[i] = std::max<int>(1, (int)(align_up((size_t)s.r_eff, 32) / 32));
      if (mode == Mode::Encode) pcj[i] = folds_mean(c, s) ? 1 : 0;   // one product form per launch
    } else if (mode == Mode::UnpackCodes) {
      key[i] = 0;
    } else {
      if (j.block_table) {
        if (j.block_size <= 0 || j.n_blocks <= 0) return fail(KVTC_E_INVALID, "job: bad paging");
        if ((size_t)j.n_blocks * j.block_size * F * out_esz > j.dst_capacity)
          return fail(KVTC_E_CAPACITY, "job: paged dst smaller than n_blocks * block_size rows");
        d.block_table = j.block_table;
        d.block_size = j.block_size;
        d.n_blocks = j.n_blocks;
      } else if ((size_t)j.n_tokens * F * out_esz > j.dst_capacity) {
        return fail(KVTC_E_CAPACITY, "job: dst smaller than n_tokens rows");
      } else {
        // Contiguous output as one block of 2^30 rows through a zero entry,
        // so the kernels have a single (paged) row mapping.
        d.block_table = c->d_zero;
        d.block_size = 1 << 30;
        d.n_blocks = 1;
      }
      if (j.block_table && (int64_t)j.n_blocks * j.block_size > (int64_t)INT32_MAX)
        return fail(KVTC_E_UNSUPPORTED, "job: paged dst has 2^31 rows or more");
      if ((d.block_size & (d.block_size - 1)) == 0)
        for (int b = 0; b < 31; ++b)
          if ((1 << b) == d.block_size) d.bs_shift = b;
      if (mode != Mode::Decode) {   // the fused decode needs no staging
        st_off[i] = st_total;
        st_total += job_staging_bytes(s, d.tc);
        if (st_total > 0 && (!d_staging || st_total > staging_bytes))
          return fail(KVTC_E_CAPACITY, "staging buffer too small");
        d.staging = d_staging + st_off[i];
      }
      key[i] = (int)(align_up((size_t)s.r_eff, 16) / 16);
      pcj[i] = s.cwidths.empty() ? 0 : 1;   // stage 1 and the fused decode take such jobs in launches of their own
      if (s.record_bytes > 24 * key[i]) return fail(KVTC_E_UNSUPPORTED, "record wider than the decode tiles");
    }
  }
  // (checked after the jobs, so job errors are reported without a device)
  if (!c->d_state || c->uploaded_version != c->calib_version)
    return fail(KVTC_E_INVALID, "device state is missing or stale: call kvtc_upload");
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int x, int y) { return key[x] != key[y] ? key[x] < key[y] : pcj[x] < pcj[y]; });
  for (int p = 0; p < n;) {
    int q = p;
    while (q < n && q - p < kMaxLaunchJobs && key[order[q]] == key[order[p]] && pcj[order[q]] == pcj[order[p]]) ++q;
    LaunchArgs a;
    std::memset(&a, 0, sizeof(a));
    a.n_jobs = q - p;
    a.dtype = c->p.dtype;
    a.out_dtype = out_dtype;
    a.F = F;
    a.state = c->d_state;
    a.status = (unsigned long long*)d_ws;
    a.sink = (uint8_t*)d_ws + sink_offset(n);
    a.epoch = next_epoch();
    a.pc = mode == Mode::Encode ? 0 : pcj[order[p]];
    a.fold = mode == Mode::Encode ? pcj[order[p]] : 0;
    uint32_t tiles = 0, cblks = 0;
    size_t rb_max = 0;
    for (int b = 0; b < a.n_jobs; ++b) {
      JobDesc d = desc[order[p + b]];
      const Slot& s = c->slots[d.slot];
      const uint32_t ptiles = (d.s1 + d.w1 + kPassRows - 1) / kPassRows;
      if (mode == Mode::Restore || mode == Mode::Decode) {
        // units: feature slabs x blocks of kDecTok tokens
        const int fs = rest_slab(rest_nfb(key[order[p]], F));
        d.n_ctiles = (uint32_t)((F + fs - 1) / fs) * ((d.tc + kDecTok - 1) / kDecTok);
      } else if (mode == Mode::Unpack) {
        d.n_ctiles = (d.tc + kDecTok - 1) / kDecTok;   // one wave per block
      } else {
        const int tile = mode == Mode::UnpackCodes ? kUnpackTile : kEncTile;
        d.n_ctiles = (d.tc + tile - 1) / tile;
      }
      d.tile_begin = tiles;
      d.cblk_begin = cblks;
      if (mode == Mode::Unpack)   // header and passthrough units
        cblks += std::max<uint32_t>(1, (d.s1 + d.w1 + kPrepPassRows - 1) / kPrepPassRows);
      else if (mode == Mode::Decode)
        cblks += std::max<uint32_t>(1, (d.s1 + d.w1 + kRestPassRows - 1) / kRestPassRows);
      else if (s.r_eff > 0)
        cblks += (d.tc + kEncBlk - 1) / kEncBlk;
      if (mode == Mode::Restore || mode == Mode::Decode || mode == Mode::Unpack || mode == Mode::UnpackCodes)
        tiles += d.n_ctiles;
      else
        tiles += std::max<uint32_t>(1, d.n_ctiles + ptiles);
      a.jobs[b] = d;
      rb_max = std::max(rb_max, (size_t)s.record_bytes);
    }
    a.total_tiles = tiles;
    a.total_cblks = cblks;
    const int k = key[order[p]];
    size_t l = 16;
    const size_t rbp = (size_t)padded_stride((int)rb_max);
    if (mode == Mode::Encode)
      l = std::max({l, enc_lds_bytes(k, F, c->p.dtype == KVTC_F32), (size_t)kEncTile * rbp});
    else if (mode == Mode::Pack)
      l = std::max(l, (size_t)kEncTile * rbp);
    else if (mode == Mode::UnpackCodes)
      l = std::max(l, (size_t)kUnpackTile * rb_max + 16);
    else if (mode == Mode::Unpack) {
      // each wave's 32 record rows, plus 16 bytes for the 8-byte reads past a row
      a.wave_lds = (uint32_t)align_up(rec_rows_bytes((int)rb_max), 16);
      l = (size_t)kPrepRowsOff + (size_t)kPrepWaves * a.wave_lds + 16;
    }
    else if (mode == Mode::Decode) {
      a.wave_lds = (uint32_t)rest_rec_bytes((int)rb_max);
      l = rest_lds_bytes(k, true, a.wave_lds);
    } else {
      l = rest_lds_bytes(k, false, 0);
    }
    if (l > 160 * 1024) return fail(KVTC_E_UNSUPPORTED, "tile does not fit in LDS");
    batches.push_back(a);
    shape.push_back(k);
    lds.push_back(l);
    p = q;
  }
  return KVTC_OK;
}

kvtc_status hip_status(int e, const char* what) {
  if (e == 0) return KVTC_OK;
  return fail(KVTC_E_HIP, std::string(what) + ": " + hipGetErrorString((hipError_t)e));
}

// Fused decode schedule: one launch per batch (headers, passthrough rows,
// dequantization and the restore), the workspace holding only the status
// words and the sink.
kvtc_status decode_fused(kvtc_codec* c, const kvtc_job* jobs, int n_jobs, int out_dtype, void* d_ws,
                         hipStream_t stream) {
  std::vector<LaunchArgs> b;
  std::vector<int> k;
  std::vector<size_t> l;
  kvtc_status st = plan(c, Mode::Decode, jobs, n_jobs, out_dtype, d_ws, nullptr, 0, b, k, l);
  if (st != KVTC_OK) return st;
  for (size_t i = 0; i < b.size(); ++i) {
    if (b[i].total_tiles + b[i].total_cblks == 0) continue;   // every job has a header unit
    st = hip_status(launch_restore(b[i], k[i], true, l[i], stream), "decode launch");
    if (st != KVTC_OK) return st;
  }
  return KVTC_OK;
}

// ---- lossless stage

// The lossless fields of a job: widths of the active groups in `act`.
LzShape lz_host_shape(const kvtc_codec* c, const Slot& s, uint32_t s1, uint32_t w1, uint32_t tc,
                      std::vector<uint8_t>& act) {
  act.clear();
  for (uint8_t b : s.widths)
    if (b) act.push_back(b);
  LzShape sh;
  sh.esz = (int)elem_bytes(c->p.dtype);
  sh.n_act = s.n_act;
  sh.G = c->p.group;
  sh.n_pt = (s1 + w1) * (uint32_t)c->F;
  sh.tc = tc;
  sh.width = act.data();
  return sh;
}

// Workspace: status words and sink, one u64 container size per job, then
// each job's region (lz_layout).
size_t lz_ws_base(int n) { return kvtc_workspace_bytes(n) + align_up(8 * (size_t)std::max(n, 1), kAlign); }

kvtc_status lz_plan(kvtc_codec* c, bool enc, const kvtc_job* jobs, int n, void* d_ws, size_t ws_bytes,
                    std::vector<LzArgs>& batches, size_t* need) {
  if (!c || !jobs || n <= 0 || n > KVTC_MAX_JOBS) return fail(KVTC_E_INVALID, "bad codec, jobs or job count");
  std::vector<LzJob> desc(n);
  std::vector<uint32_t> units(n), segs(n), nfs(n), chunks(n);
  std::vector<int> rbs(n);
  std::vector<uint8_t> act;
  size_t off = lz_ws_base(n);
  for (int i = 0; i < n; ++i) {
    const kvtc_job& j = jobs[i];
    int idx;
    if (!slot_index(c, j.layer, j.kind, &idx)) return fail(KVTC_E_INVALID, "job: bad layer or kind");
    const Slot& s = c->slots[idx];
    if (!s.calibrated) return fail(KVTC_E_NOT_CALIBRATED, "job: (layer, kind) is not calibrated");
    if (j.n_tokens < 0 || j.n_tokens > (int64_t)INT32_MAX) return fail(KVTC_E_INVALID, "job: bad n_tokens");
    LzJob& d = desc[i];
    std::memset(&d, 0, sizeof(d));
    d.T = (uint32_t)j.n_tokens;
    split_rows(j.n_tokens, c->p, &d.s1, &d.w1, &d.tc);
    const LzShape sh = lz_host_shape(c, s, d.s1, d.w1, d.tc, act);
    const LzLayout L = lz_layout(sh, enc);
    const size_t sb = stream_bytes(c, s, j.n_tokens), bound = lz_bound(sh);
    if (bound >= (1ull << 32) - 16) return fail(KVTC_E_UNSUPPORTED, "job: container could reach 4 GiB");
    if (!need) {
      if (!j.src || !aligned16(j.src) || !j.dst || !aligned16(j.dst))
        return fail(KVTC_E_INVALID, "job: src and dst must be non-null and 16-byte aligned");
      if (enc && j.src_capacity < sb) return fail(KVTC_E_CAPACITY, "job: src_capacity below kvtc_encoded_bytes");
      if (enc && j.dst_capacity < bound) return fail(KVTC_E_CAPACITY, "job: dst_capacity below kvtc_lossless_bound");
      if (!enc && j.src_capacity < L.pay_off) return fail(KVTC_E_CAPACITY, "job: src_capacity below the container's tables");
      if (!enc && j.dst_capacity < sb) return fail(KVTC_E_CAPACITY, "job: dst_capacity below kvtc_encoded_bytes");
    }
    d.src = (const uint8_t*)j.src;
    d.dst = (uint8_t*)j.dst;
    d.ws = (uint8_t*)d_ws + off;
    d.src_cap = j.src_capacity;
    d.stream_bytes = sb;
    d.slot = idx;
    d.status_idx = i;
    off += L.bytes;
    units[i] = std::max<uint32_t>(1, (sh.n_pt + kLzPassBlk - 1) / kLzPassBlk + (d.tc + kLzRecBlk - 1) / kLzRecBlk);
    segs[i] = L.n_segs;
    nfs[i] = (uint32_t)lz_nf(sh);
    chunks[i] = L.n_chunks;
    rbs[i] = s.record_bytes;
  }
  if (need) {
    *need = off;
    return KVTC_OK;
  }
  if (!d_ws || !aligned16(d_ws)) return fail(KVTC_E_INVALID, "workspace must be non-null and aligned");
  if (ws_bytes < off) return fail(KVTC_E_CAPACITY, "workspace below kvtc_lossless_workspace_bytes");
  if (!c->d_state || c->uploaded_version != c->calib_version)
    return fail(KVTC_E_INVALID, "device state is missing or stale: call kvtc_upload");
  for (int p = 0; p < n; p += kMaxLaunchJobs) {
    LzArgs a;
    std::memset(&a, 0, sizeof(a));
    a.n_jobs = std::min(n - p, kMaxLaunchJobs);
    a.esz = (int)elem_bytes(c->p.dtype);
    a.F = c->F;
    a.state = c->d_state;
    a.status = (unsigned long long*)d_ws;
    a.sizes = (unsigned long long*)((uint8_t*)d_ws + kvtc_workspace_bytes(n));
    a.epoch = next_epoch();
    int rb_max = 0;
    for (int b = 0; b < a.n_jobs; ++b) {
      LzJob d = desc[p + b];
      d.unit0 = a.units;
      d.seg0 = a.segs;
      d.field0 = a.fields;
      d.chunk0 = a.chunks;
      a.units += units[p + b];
      a.segs += segs[p + b];
      a.fields += nfs[p + b];
      a.chunks += chunks[p + b];
      rb_max = std::max(rb_max, rbs[p + b]);
      a.jobs[b] = d;
    }
    a.rec_lds = (size_t)kLzRecBlk * rb_max + 16;   // split: the block's records; merge: its symbols
    for (int b = 0; b < a.n_jobs; ++b) {
      const Slot& sl = c->slots[a.jobs[b].slot];
      a.rec_lds = std::max(a.rec_lds, (size_t)kLzRecBlk * sl.n_act * (8 + c->p.group) + 16);
    }
    batches.push_back(a);
  }
  return KVTC_OK;
}

}  // namespace

extern "C" {

kvtc_status kvtc_encode(kvtc_codec* c, const kvtc_job* jobs, int32_t n_jobs, void* d_ws,
                        hipStream_t stream) {
  std::vector<LaunchArgs> b;
  std::vector<int> k;
  std::vector<size_t> l;
  kvtc_status st = plan(c, Mode::Encode, jobs, n_jobs, c ? c->p.dtype : 0, d_ws, nullptr, 0, b, k, l);
  if (st != KVTC_OK) return st;
  for (size_t i = 0; i < b.size(); ++i) {
    if (b[i].total_tiles == 0) continue;
    st = hip_status(launch_encode(b[i], k[i], c->p.group, l[i], stream), "encode launch");
    if (st != KVTC_OK) return st;
  }
  return KVTC_OK;
}

kvtc_status kvtc_decode_unpack(kvtc_codec* c, const kvtc_job* jobs, int32_t n_jobs, int32_t out_dtype,
                               void* d_staging, size_t staging_bytes, void* d_ws, hipStream_t stream) {
  std::vector<LaunchArgs> b;
  std::vector<int> k;
  std::vector<size_t> l;
  kvtc_status st = plan(c, Mode::Unpack, jobs, n_jobs, out_dtype, d_ws, (uint8_t*)d_staging,
                        staging_bytes, b, k, l);
  if (st != KVTC_OK) return st;
  for (size_t i = 0; i < b.size(); ++i) {
    if (b[i].total_tiles + b[i].total_cblks == 0) continue;   // every job has a header unit
    st = hip_status(launch_prep(b[i], k[i], l[i], stream), "decode stage 1 launch");
    if (st != KVTC_OK) return st;
  }
  return KVTC_OK;
}

kvtc_status kvtc_decode_restore(kvtc_codec* c, const kvtc_job* jobs, int32_t n_jobs, int32_t out_dtype,
                                const void* d_staging, size_t staging_bytes, void* d_ws,
                                hipStream_t stream) {
  std::vector<LaunchArgs> b;
  std::vector<int> k;
  std::vector<size_t> l;
  kvtc_status st = plan(c, Mode::Restore, jobs, n_jobs, out_dtype, d_ws, (uint8_t*)d_staging,
                        staging_bytes, b, k, l);
  if (st != KVTC_OK) return st;
  for (size_t i = 0; i < b.size(); ++i) {
    if (b[i].total_tiles == 0) continue;
    st = hip_status(launch_restore(b[i], k[i], false, l[i], stream), "decode stage 2 launch");
    if (st != KVTC_OK) return st;
  }
  return KVTC_OK;
}

kvtc_status kvtc_decode(kvtc_codec* c, const kvtc_job* jobs, int32_t n_jobs, int32_t out_dtype,
                        void* d_ws, size_t ws_bytes, hipStream_t stream) {
  if (!c || !jobs || n_jobs <= 0 || n_jobs > KVTC_MAX_JOBS) return fail(KVTC_E_INVALID, "bad codec, jobs or job count");
  const size_t need = kvtc_decode_workspace_bytes(c, jobs, n_jobs);
  if (need == 0) return fail(KVTC_E_INVALID, "job: bad layer or kind, or not calibrated");
  const size_t base = kvtc_workspace_bytes(n_jobs);
  if (!d_ws || ws_bytes < base) return fail(KVTC_E_CAPACITY, "workspace below kvtc_workspace_bytes(n_jobs)");
  if (ws_bytes >= need) {
    // Two-stage schedule, the staging right after the status words and sink.
    // Stage 2 of each batch follows its stage 1, so the batch's staging is
    // still in the caches when it is read back. (Both plans group the jobs
    // by K-step count the same way, so their batches correspond.)
    uint8_t* stg = need > base ? (uint8_t*)d_ws + base : nullptr;
    std::vector<LaunchArgs> bu, br;
    std::vector<int> ku, kr;
    std::vector<size_t> lu, lr;
    kvtc_status st = plan(c, Mode::Unpack, jobs, n_jobs, out_dtype, d_ws, stg, need - base, bu, ku, lu);
    if (st != KVTC_OK) return st;
    st = plan(c, Mode::Restore, jobs, n_jobs, out_dtype, d_ws, stg, need - base, br, kr, lr);
    if (st != KVTC_OK) return st;
    if (bu.size() != br.size()) return fail(KVTC_E_INVALID, "internal: stage batches differ");
    for (size_t i = 0; i < bu.size(); ++i) {
      if (bu[i].total_tiles + bu[i].total_cblks > 0) {   // every job has a header unit
        st = hip_status(launch_prep(bu[i], ku[i], lu[i], stream), "decode stage 1 launch");
        if (st != KVTC_OK) return st;
      }
      if (br[i].total_tiles > 0) {
        st = hip_status(launch_restore(br[i], kr[i], false, lr[i], stream), "decode stage 2 launch");
        if (st != KVTC_OK) return st;
      }
    }
    return KVTC_OK;
  }
  return decode_fused(c, jobs, n_jobs, out_dtype, d_ws, stream);
}

kvtc_status kvtc_decode_noalloc(kvtc_codec* c, const kvtc_job* jobs, int32_t n_jobs, int32_t out_dtype,
                                int32_t* d_status, hipStream_t stream) {
  if (!c || !jobs || n_jobs <= 0) return fail(KVTC_E_INVALID, "bad codec, jobs or job count");
  void* ws = nullptr;
  size_t ws_cap = 0;
  kvtc_status st = hip_status(noalloc_scratch(&ws, &ws_cap), "static workspace lookup");
  if (st != KVTC_OK) return st;
  if (kvtc_workspace_bytes(n_jobs) > ws_cap)
    return fail(KVTC_E_CAPACITY, "more jobs than kvtc_decode_noalloc's static workspace holds (KVTC_MAX_JOBS)");
  if (kvtc_decode_workspace_bytes(c, jobs, n_jobs) == 0)
    return fail(KVTC_E_INVALID, "job: bad layer or kind, or not calibrated");
  // the array keeps the last call's words: start this call's from zero
  st = hip_status(launch_clear_words(ws, n_jobs, stream), "status clear launch");
  if (st != KVTC_OK) return st;
  st = decode_fused(c, jobs, n_jobs, out_dtype, ws, stream);
  if (st != KVTC_OK || !d_status) return st;
  return hip_status(launch_status_codes(ws, d_status, n_jobs, stream), "status launch");
}

kvtc_status kvtc_unpack(kvtc_codec* c, const kvtc_job* job, void* d_codes, void* d_shift_scale, void* d_ws,
                        hipStream_t stream) {
  std::vector<LaunchArgs> b;
  std::vector<int> k;
  std::vector<size_t> l;
  kvtc_status st = plan(c, Mode::UnpackCodes, job, 1, c ? c->p.dtype : 0, d_ws, nullptr, 0, b, k, l);
  if (st != KVTC_OK) return st;
  const int idx = job->layer * 2 + job->kind;
  if (c->slots[idx].r_eff > 0 && (!d_codes || !d_shift_scale))
    return fail(KVTC_E_INVALID, "null codes or shift/scale");
  for (size_t i = 0; i < b.size(); ++i) {
    if (b[i].total_tiles == 0) continue;
    st = hip_status(launch_unpack(b[i], c->p.group, l[i], d_codes, d_shift_scale, stream), "unpack launch");
    if (st != KVTC_OK) return st;
  }
  return KVTC_OK;
}

kvtc_status kvtc_pack(kvtc_codec* c, const kvtc_job* job, const void* d_codes, const void* d_shift_scale,
                      void* d_ws, hipStream_t stream) {
  std::vector<LaunchArgs> b;
  std::vector<int> k;
  std::vector<size_t> l;
  kvtc_status st = plan(c, Mode::Pack, job, 1, c ? c->p.dtype : 0, d_ws, nullptr, 0, b, k, l);
  if (st != KVTC_OK) return st;
  int idx = job->layer * 2 + job->kind;
  if (c->slots[idx].r_eff > 0 && (!d_codes || !d_shift_scale))
    return fail(KVTC_E_INVALID, "null codes or shift/scale");
  return hip_status(launch_pack(b[0], c->p.group, l[0], d_codes, d_shift_scale, stream), "pack launch");
}

kvtc_status kvtc_read_device_status(const void* d_ws, int32_t n_jobs, int32_t* status, hipStream_t stream) {
  if (!d_ws || !status || n_jobs <= 0) return fail(KVTC_E_INVALID, "bad arguments");
  std::vector<uint64_t> words(n_jobs);
  hipError_t e = hipStreamSynchronize(stream);
  if (e == hipSuccess) e = hipMemcpy(words.data(), d_ws, sizeof(uint64_t) * n_jobs, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(KVTC_E_HIP, std::string("status read: ") + hipGetErrorString(e));
  for (int i = 0; i < n_jobs; ++i) status[i] = rank_status((int)(words[i] & 0xFF));
  return KVTC_OK;
}

size_t kvtc_lossless_bound(const kvtc_codec* c, int32_t layer, int32_t kind, int64_t n_tokens) {
  int idx;
  if (!slot_index(c, layer, kind, &idx) || n_tokens < 0 || !c->slots[idx].calibrated) return 0;
  uint32_t s1, w1, tc;
  split_rows(n_tokens, c->p, &s1, &w1, &tc);
  std::vector<uint8_t> act;
  return lz_bound(lz_host_shape(c, c->slots[idx], s1, w1, tc, act));
}

size_t kvtc_lossless_workspace_bytes(const kvtc_codec* c, const kvtc_job* jobs, int32_t n_jobs, int32_t encode) {
  std::vector<LzArgs> b;
  size_t need = 0;
  if (lz_plan(const_cast<kvtc_codec*>(c), encode != 0, jobs, n_jobs, nullptr, 0, b, &need) != KVTC_OK) return 0;
  return need;
}

kvtc_status kvtc_lossless_encode(kvtc_codec* c, const kvtc_job* jobs, int32_t n_jobs, void* d_ws,
                                 size_t ws_bytes, hipStream_t stream) {
  std::vector<LzArgs> b;
  kvtc_status st = lz_plan(c, true, jobs, n_jobs, d_ws, ws_bytes, b, nullptr);
  if (st != KVTC_OK) return st;
  for (const LzArgs& a : b) {
    st = hip_status(launch_lz_encode(a, stream), "lossless encode launch");
    if (st != KVTC_OK) return st;
  }
  return KVTC_OK;
}

kvtc_status kvtc_lossless_decode(kvtc_codec* c, const kvtc_job* jobs, int32_t n_jobs, void* d_ws,
                                 size_t ws_bytes, hipStream_t stream) {
  std::vector<LzArgs> b;
  kvtc_status st = lz_plan(c, false, jobs, n_jobs, d_ws, ws_bytes, b, nullptr);
  if (st != KVTC_OK) return st;
  for (const LzArgs& a : b) {
    st = hip_status(launch_lz_decode(a, stream), "lossless decode launch");
    if (st != KVTC_OK) return st;
  }
  return KVTC_OK;
}

kvtc_status kvtc_lossless_sizes(const void* d_ws, int32_t n_jobs, uint64_t* sizes, hipStream_t stream) {
  if (!d_ws || !sizes || n_jobs <= 0) return fail(KVTC_E_INVALID, "bad arguments");
  hipError_t e = hipStreamSynchronize(stream);
  if (e == hipSuccess)
    e = hipMemcpy(sizes, (const uint8_t*)d_ws + kvtc_workspace_bytes(n_jobs), sizeof(uint64_t) * n_jobs,
                  hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(KVTC_E_HIP, std::string("container sizes read: ") + hipGetErrorString(e));
  return KVTC_OK;
}

kvtc_status kvtc_deflate(const void* in, size_t n, void* out, size_t cap, size_t* out_len, int32_t level) {
  if ((!in && n) || !out_len) return fail(KVTC_E_INVALID, "bad arguments");
  const uLong bound = compressBound((uLong)n);
  if (!out) {
    *out_len = bound;
    return KVTC_OK;
  }
  uLongf len = (uLongf)cap;
  const int z = compress2((Bytef*)out, &len, (const Bytef*)in, (uLong)n, level);
  if (z == Z_BUF_ERROR) return fail(KVTC_E_CAPACITY, "deflate output buffer too small");
  if (z != Z_OK) return fail(KVTC_E_INVALID, "zlib error");
  *out_len = len;
  return KVTC_OK;
}

}  // extern "C"
