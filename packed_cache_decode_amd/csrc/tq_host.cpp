// Host side of the TurboQuant packed KV-cache library: the C ABI of
// include/tq.h, the codebook solver, the rotation signs, argument validation
// and kernel launches.
//
// Sources (page title, section):
//   P1 "vLLM 源码完全拆解(十九):TurboQuant KV Cache 量化" -- presets ("四个
//      预设对应什么"), Lloyd-Max conditions and the page's numerical recipe
//      ("Lloyd-Max 的两个最优性条件", "vLLM 的实现:数值积分而不是解析解"),
//      midpoints ("vLLM 内置的 Lloyd-Max 码本"), slot arithmetic ("从
//      slot_size 的三项算术开始"), paging ("页内寻址").
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <limits>
#include <mutex>
#include <vector>

#include "tq_internal.h"

using tq::DevTables;
using tq::DevErrors;
using tq::Geometry;

struct tq_ctx {
  int preset;
  int codebook_mode;
  Geometry geo;
  int levels;                       // 2^key_bits for MSE keys, 0 for fp8
  float centroids[tq::kMaxLevels];
  float midpoints[tq::kMaxLevels];
  int8_t signs[tq::kMaxHeadDim];
  float r_d;                        // float32(1 / sqrt(head_dim))
  int device;
  DevTables* d_tables;              // read-only to the kernels
  DevErrors* d_errs;                // sticky error words, written by the kernels
  float* d_rot;                     // Haar rotation matrix (device), or null
  tq_decode_options opts;           // decode plan options (tq_set_decode_options)
  void* scratch;                    // this device's allocation-free decode scratch
};

// ---- scratch of the allocation-free decode --------------------------------
// tq_decode_noalloc keeps its split partials in this file-scope device array
// instead of a caller workspace: each GPU the library runs on holds its own
// copy until the process ends.  In host code the array's name is not a device
// address; the address of a device's copy comes from hipGetSymbolAddress,
// taken once per device with that device current (in tq_codebook_init), and
// only that address is passed to kernels.
constexpr size_t kNoAllocScratchBytes = size_t{32} << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// this device's copy of the scratch array (the device must be current);
// null if its address cannot be taken
void* noalloc_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[device] = p;
  }
  return g_scratch_ptr[device];
}

// ---- Lloyd-Max for N(0, sigma^2) ------------------------------------------
// Fixed point of the two optimality conditions: boundaries at midpoints of
// neighbouring levels, levels at the conditional mean of their cell, the
// outer cells open to +-infinity.  Conditional mean of a Gaussian over (a, b):
//   sigma * (phi(a/sigma) - phi(b/sigma)) / (Phi(b/sigma) - Phi(a/sigma)).

double std_pdf(double z) {
  if (std::isinf(z)) return 0.0;
  return std::exp(-0.5 * z * z) / std::sqrt(2.0 * M_PI);
}

// P(a < Z < b) for a standard normal Z, from whichever tail keeps precision.
double std_mass(double a, double b) {
  const double r2 = std::sqrt(2.0);
  if (a >= 0.0) return 0.5 * (std::erfc(a / r2) - std::erfc(b / r2));
  if (b <= 0.0) return 0.5 * (std::erfc(-b / r2) - std::erfc(-a / r2));
  return 1.0 - 0.5 * std::erfc(-a / r2) - 0.5 * std::erfc(b / r2);
}

double cell_mean(double a, double b, double sigma) {
  const double za = a / sigma, zb = b / sigma;
  return sigma * (std_pdf(za) - std_pdf(zb)) / std_mass(za, zb);
}

bool solve_exact(int d, int bits, std::vector<double>& out) {
  const int n = 1 << bits;
  const double sigma = std::sqrt(1.0 / d);
  const double lo = -3.5 * sigma, hi = 3.5 * sigma;
  std::vector<double> c(n), nc(n), edges(n + 1);
  for (int i = 0; i < n; ++i) c[i] = lo + (hi - lo) * (i + 0.5) / n;
  bool converged = false;
  for (int it = 0; it < 100000 && !converged; ++it) {
    edges[0] = -INFINITY;
    edges[n] = INFINITY;
    for (int i = 0; i + 1 < n; ++i) edges[i + 1] = (c[i] + c[i + 1]) / 2.0;
    double delta = 0.0;
    for (int i = 0; i < n; ++i) {
      nc[i] = cell_mean(edges[i], edges[i + 1], sigma);
      delta = std::fmax(delta, std::fabs(nc[i] - c[i]));
    }
    c.swap(nc);
    converged = delta < 1e-14;
  }
  if (!converged) return false;
  // exact symmetry: mirror the positive half
  out.assign(n, 0.0);
  for (int i = 0; i < n / 2; ++i) {
    out[n / 2 + i] = c[n / 2 + i];
    out[n / 2 - 1 - i] = -c[n / 2 + i];
  }
  return true;
}

// ---- the page's numerical recipe ----------------------------------------
// From the parameters the page states: levels start evenly spread over
// +-3.5 sigma; the outer cells end at +-10.5 sigma instead of +-infinity;
// each cell's mass and first moment come from the composite trapezoid rule on
// 200 equal panels; the iteration stops as soon as an update would move no
// level by 1e-10 or more (keeping the levels it had), or after 200 updates.
// Sums run in node order, so the tables equal the test oracle's bit for bit.
constexpr int kPagePanels = 200;
constexpr double kPageOuterSigmas = 10.5;
constexpr double kPageTol = 1e-10;
constexpr int kPageMaxIter = 200;

double gauss_density(double x, double var) {
  return std::exp(-x * x / (2.0 * var)) / std::sqrt(2.0 * M_PI * var);
}

// (mass, first moment) of N(0, var) over [a, b]: nodes a + j h, weight h
// (h / 2 at both ends)
void trapezoid_cell_moments(double a, double b, double var, double& mass, double& first) {
  const double h = (b - a) / kPagePanels;
  double m = 0.0, f = 0.0;
  for (int j = 0; j <= kPagePanels; ++j) {
    const double x = a + j * h;
    double fx = gauss_density(x, var);
    if (j == 0 || j == kPagePanels) fx = 0.5 * fx;
    m += fx;
    f += x * fx;
  }
  mass = m * h;
  first = f * h;
}

void solve_page_trapz(int d, int bits, std::vector<double>& levels) {
  const int n = 1 << bits;
  const double var = 1.0 / d;
  const double sigma = std::sqrt(var);
  const double outer = kPageOuterSigmas * sigma;
  const double lo = -3.5 * sigma, hi = 3.5 * sigma;
  levels.assign(n, 0.0);
  for (int i = 0; i < n; ++i) levels[i] = lo + (hi - lo) * (i + 0.5) / n;
  std::vector<double> bounds(n + 1), means(n);
  for (int it = 0; it < kPageMaxIter; ++it) {
    bounds[0] = -outer;
    bounds[n] = outer;
    for (int i = 1; i < n; ++i) bounds[i] = (levels[i - 1] + levels[i]) / 2.0;
    double moved = 0.0;
    for (int i = 0; i < n; ++i) {
      double mass, first;
      trapezoid_cell_moments(bounds[i], bounds[i + 1], var, mass, first);
      means[i] = first / mass;          // every cell has positive mass here
      moved = std::fmax(moved, std::fabs(means[i] - levels[i]));
    }
    if (moved < kPageTol) return;
    levels.swap(means);
  }
}

// ---- Lloyd-Max for the exact sphere marginal --------------------------------
// One coordinate of a uniformly random unit vector in R^d has density
// proportional to (1 - x^2)^((d-3)/2) on [-1, 1] (a scaled Beta law).  Cell
// masses and first moments by composite Gauss-Legendre quadrature (32 nodes
// on each of 32 equal panels of the cell); the same fixed point as
// solve_exact with the outer cells ending at -1 and +1.

// nodes and weights of the n-point Gauss-Legendre rule on [-1, 1], by Newton's
// method on the Legendre polynomial P_n (three-term recurrence)
void gauss_legendre(int n, std::vector<double>& x, std::vector<double>& w) {
  x.assign(n, 0.0);
  w.assign(n, 0.0);
  for (int i = 0; i < (n + 1) / 2; ++i) {
    double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
    double dp = 0.0;
    for (int it = 0; it < 100; ++it) {
      double p0 = 1.0, p1 = z;
      for (int k = 2; k <= n; ++k) {
        const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
        p0 = p1;
        p1 = p2;
      }
      dp = n * (z * p1 - p0) / (z * z - 1.0);
      const double dz = p1 / dp;
      z -= dz;
      if (std::fabs(dz) < 1e-16) break;
    }
    x[i] = -z;
    x[n - 1 - i] = z;
    w[i] = w[n - 1 - i] = 2.0 / ((1.0 - z * z) * dp * dp);
  }
}

bool solve_beta(int d, int bits, std::vector<double>& out) {
  const int n = 1 << bits;
  const double a = (d - 3) / 2.0;
  std::vector<double> gx, gw;
  gauss_legendre(32, gx, gw);
  auto moments = [&](double l, double u, double& m0, double& m1) {
    const int panels = 32;
    const double h = (u - l) / panels;
    m0 = m1 = 0.0;
    for (int p = 0; p < panels; ++p) {
      const double mid = l + (p + 0.5) * h;
      for (size_t k = 0; k < gx.size(); ++k) {
        const double x = mid + 0.5 * h * gx[k];
        const double f = std::pow(std::fmax(1.0 - x * x, 0.0), a) * gw[k] * 0.5 * h;
        m0 += f;
        m1 += x * f;
      }
    }
  };
  const double spread = std::fmin(3.5 * std::sqrt(1.0 / d), 1.0);
  std::vector<double> c(n), nc(n), edges(n + 1);
  for (int i = 0; i < n; ++i) c[i] = -spread + 2.0 * spread * (i + 0.5) / n;
  bool converged = false;
  for (int it = 0; it < 100000 && !converged; ++it) {
    edges[0] = -1.0;
    edges[n] = 1.0;
    for (int i = 0; i + 1 < n; ++i) edges[i + 1] = (c[i] + c[i + 1]) / 2.0;
    double delta = 0.0;
    for (int i = 0; i < n; ++i) {
      double m0, m1;
      moments(edges[i], edges[i + 1], m0, m1);
      nc[i] = m1 / m0;
      delta = std::fmax(delta, std::fabs(nc[i] - c[i]));
    }
    c.swap(nc);
    converged = delta < 1e-14;
  }
  if (!converged) return false;
  out.assign(n, 0.0);
  for (int i = 0; i < n / 2; ++i) {
    out[n / 2 + i] = c[n / 2 + i];
    out[n / 2 - 1 - i] = -c[n / 2 + i];
  }
  return true;
}

// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): sign j is the top bit of
// the j-th output, 1 -> -1.
void rotation_signs(uint64_t seed, int d, bool flip, int8_t* s) {
  uint64_t st = seed;
  for (int j = 0; j < d; ++j) {
    if (!flip) {
      s[j] = 1;
      continue;
    }
    st += 0x9E3779B97F4A7C15ull;
    uint64_t z = st;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    s[j] = (z >> 63) ? -1 : 1;
  }
}

// ---- Haar rotation ------------------------------------------------------------
// Gaussian entries from the SplitMix64 stream of rot_seed: uniforms
// u = ((z >> 11) + 1/2) 2^-53, Box-Muller on consecutive pairs; G filled row by
// row.  Householder QR of G, then Q diag(sign(diag R)) (Mezzadri 2007), which
// is Haar distributed; rounded to float32.
void haar_matrix(uint64_t seed, int d, std::vector<float>& q32) {
  const int n = d * d;
  std::vector<double> g(n + (n & 1));
  uint64_t st = seed;
  auto next = [&]() {
    st += 0x9E3779B97F4A7C15ull;
    uint64_t z = st;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (static_cast<double>(z >> 11) + 0.5) / 9007199254740992.0;
  };
  for (size_t m = 0; m < g.size(); m += 2) {
    const double u1 = next(), u2 = next();
    const double r = std::sqrt(-2.0 * std::log(u1));
    g[m] = r * std::cos(2.0 * M_PI * u2);
    g[m + 1] = r * std::sin(2.0 * M_PI * u2);
  }
  // A = G (row-major); Householder: for column k, v = x + sign(x0)|x| e0 on rows k..d-1
  std::vector<double> A(g.begin(), g.begin() + n), V(n, 0.0), beta(d, 0.0), rdiag(d, 0.0);
  for (int k = 0; k < d; ++k) {
    double norm = 0.0;
    for (int i = k; i < d; ++i) norm += A[i * d + k] * A[i * d + k];
    norm = std::sqrt(norm);
    const double x0 = A[k * d + k];
    const double alpha = x0 >= 0.0 ? -norm : norm;        // R[k][k]
    rdiag[k] = alpha;
    double vnorm2 = 0.0;
    for (int i = k; i < d; ++i) {
      V[i * d + k] = A[i * d + k] - (i == k ? alpha : 0.0);
      vnorm2 += V[i * d + k] * V[i * d + k];
    }
    beta[k] = vnorm2 > 0.0 ? 2.0 / vnorm2 : 0.0;
    // apply H_k = I - beta v v^T to the remaining columns
    for (int j = k; j < d; ++j) {
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += V[i * d + k] * A[i * d + j];
      dot *= beta[k];
      for (int i = k; i < d; ++i) A[i * d + j] -= dot * V[i * d + k];
    }
  }
  // Q = H_0 H_1 ... H_{d-1} applied to the identity, from the last reflector
  std::vector<double> Q(n, 0.0);
  for (int i = 0; i < d; ++i) Q[i * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k)
    for (int j = 0; j < d; ++j) {
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += V[i * d + k] * Q[i * d + j];
      dot *= beta[k];
      for (int i = k; i < d; ++i) Q[i * d + j] -= dot * V[i * d + k];
    }
  q32.assign(n, 0.0f);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      const double sgn = rdiag[j] < 0.0 ? -1.0 : 1.0;      // sign of R[j][j]
      q32[i * d + j] = static_cast<float>(Q[i * d + j] * sgn);
    }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

tq_status check_device(const tq_ctx* ctx) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return TQ_ERR_NO_DEVICE;
  if (dev != ctx->device) return TQ_ERR_INVALID_ARG;
  return TQ_OK;
}

// float32 levels (ascending) and midpoints of the sorted float32 levels,
// m_i = (c_i + c_{i+1}) / 2 in float32.
tq_status host_codebook(int d, int bits, int mode, float* cent, float* mid) {
  if (bits < 1 || bits > 4) return TQ_ERR_UNSUPPORTED;
  std::vector<double> lv;
  if (mode == TQ_CODEBOOK_LLOYD_MAX_EXACT) {
    if (!solve_exact(d, bits, lv)) return TQ_ERR_UNSUPPORTED;
  } else if (mode == TQ_CODEBOOK_PAGE_TRAPZ) {
    solve_page_trapz(d, bits, lv);
  } else if (mode == TQ_CODEBOOK_BETA_EXACT) {
    if (!solve_beta(d, bits, lv)) return TQ_ERR_UNSUPPORTED;
  } else {
    return TQ_ERR_INVALID_ARG;
  }
  std::vector<float> f(lv.size());
  for (size_t i = 0; i < lv.size(); ++i) f[i] = static_cast<float>(lv[i]);
  for (size_t i = 1; i < f.size(); ++i)
    for (size_t j = i; j > 0 && f[j - 1] > f[j]; --j) std::swap(f[j - 1], f[j]);
  const int n = 1 << bits;
  for (int i = 0; i < n; ++i) cent[i] = f[i];
  for (int i = 0; i + 1 < n; ++i) mid[i] = (f[i] + f[i + 1]) / 2.0f;
  return TQ_OK;
}

// The device's bin arithmetic, replayed on the host (IEEE fmaf and floorf
// give the device's results): the code of y from the bins of t.
uint32_t bin_code(const DevTables& t, float y) {
  const float f = std::floor(std::fmaf(y, t.bin_scale, t.bin_bias));
  int i = std::isnan(f) ? 0 : (f < 0.0f ? 0 : (f > static_cast<float>(t.bin_count - 1) ? t.bin_count - 1
                                                                                       : static_cast<int>(f)));
  float thr;
  std::memcpy(&thr, &t.bins[i][0], 4);
  return t.bins[i][1] + (y >= thr ? 1u : 0u);
}

// Bucketize bins for midpoints mid[0..n_mid-1] (ascending fp32): see
// DevTables.  Bin j covers [(j + phi) / 2^k, (j + 1 + phi) / 2^k): 2^-k is at
// most the smallest midpoint gap, and the offset phi keeps every midpoint
// (the central one is 0) clear of the edges by 4x the fma's rounding error.
// The table is then checked against the count on every midpoint, its float
// neighbours and every edge's neighbours.  Returns false if no (k, phi)
// works within kMaxBins bins.
bool build_bins(const float* mid, int n_mid, DevTables& t) {
  double min_gap = 1e30;
  for (int i = 0; i + 1 < n_mid; ++i) min_gap = std::min(min_gap, static_cast<double>(mid[i + 1]) - mid[i]);
  if (!(min_gap > 0)) return false;
  int k0 = 0;
  while (std::ldexp(1.0, -k0) > min_gap) ++k0;
  // a bin without a midpoint gets a NaN threshold: y >= NaN is false for
  // every y, +inf included
  const float inf = std::numeric_limits<float>::infinity();
  const float none = std::numeric_limits<float>::quiet_NaN();
  uint32_t none_bits;
  std::memcpy(&none_bits, &none, 4);
  const double phis[] = {0.5, 0.25, 0.75, 0.125, 0.375, 0.625, 0.875};
  for (int k = k0; k <= k0 + 2; ++k) {
    for (double phi : phis) {
      const double w = std::ldexp(1.0, -k);
      const long jlo = static_cast<long>(std::floor(mid[0] / w - phi)) - 1;
      const long jhi = static_cast<long>(std::floor(mid[n_mid - 1] / w - phi)) + 1;
      const long count = jhi - jlo + 2;                // bin 0 + bins jlo .. jhi
      if (count > tq::kMaxBins) continue;
      // fma(y, 2^k, bias) below 2^6 in magnitude is off by at most 2^-19
      const double margin = std::ldexp(1.0, -17 - k);
      bool clear = true;
      for (int i = 0; i < n_mid && clear; ++i) {
        const double e = (std::round(mid[i] / w - phi) + phi) * w;   // nearest edge
        if (std::fabs(static_cast<double>(mid[i]) - e) <= margin) clear = false;
      }
      if (!clear) continue;
      DevTables c = t;
      std::memset(c.bins, 0, sizeof(c.bins));
      c.bins[0][0] = none_bits;
      c.bins[0][1] = 0;
      for (long j = jlo; j <= jhi; ++j) {
        const double e = (j + phi) * w;
        uint32_t base = 0;
        float thr = none;
        for (int i = 0; i < n_mid; ++i) {
          if (mid[i] <= e) ++base;
          else if (mid[i] < e + w) thr = mid[i];
        }
        std::memcpy(&c.bins[j - jlo + 1][0], &thr, 4);
        c.bins[j - jlo + 1][1] = base;
      }
      c.bin_count = static_cast<int32_t>(count);
      c.bin_scale = static_cast<float>(std::ldexp(1.0, k));
      c.bin_bias = static_cast<float>(1 - jlo - phi);
      // check: midpoints, their neighbours, edges' neighbours, zeros, NaN, +-inf
      std::vector<float> probe = {0.0f, -0.0f, inf, -inf, std::numeric_limits<float>::quiet_NaN(),
                                  1e30f, -1e30f};
      for (int i = 0; i < n_mid; ++i) {
        probe.push_back(mid[i]);
        probe.push_back(std::nextafter(mid[i], inf));
        probe.push_back(std::nextafter(mid[i], -inf));
      }
      for (long j = jlo - 1; j <= jhi + 2; ++j) {
        const float e = static_cast<float>((j + phi) * w);
        float lo = e, hi = e;
        for (int r = 0; r < 4; ++r) {
          probe.push_back(lo);
          probe.push_back(hi);
          lo = std::nextafter(lo, -inf);
          hi = std::nextafter(hi, inf);
        }
      }
      bool ok = true;
      for (float y : probe) {
        uint32_t want = 0;
        for (int i = 0; i < n_mid; ++i) want += y >= mid[i] ? 1u : 0u;
        if (bin_code(c, y) != want) ok = false;
      }
      if (!ok) continue;
      t = c;
      return true;
    }
  }
  return false;
}

int key_bits_of(int preset) { return preset == TQ_K8V4 ? 8 : (preset == TQ_4BIT_NC ? 4 : 3); }
int value_bits_of(int preset) { return preset == TQ_3BIT_NC ? 3 : 4; }

int slot_bytes_for(int preset, int d) {
  const int kb = key_bits_of(preset);
  const int key = kb == 8 ? d : (d * kb + 7) / 8 + 2;
  const int s = key + (d * value_bits_of(preset) + 7) / 8 + 4;
  return s + (s % 2);
}

}  // namespace

namespace {
// tq_decode's checks, plan and launch, with the split partials in
// `workspace` (workspace_bytes long): the caller's buffer, or the
// allocation-free entry point's scratch array
tq_status decode_impl(const tq_ctx* ctx, const void* q, const uint8_t* cache, int64_t num_blocks,
                    const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                    int batch, int num_q_heads, int max_seq_len, float sm_scale, void* out,
                    int out_is_fp32, void* workspace, size_t workspace_bytes, void* stream) {
  if (!ctx) return TQ_ERR_INVALID_ARG;
  const Geometry& g = ctx->geo;
  if (batch < 0 || num_q_heads <= 0 || max_seq_len < 0 || num_blocks < 0 ||
      max_blocks_per_seq < 0)
    return TQ_ERR_INVALID_ARG;
  if (num_q_heads % g.num_kv_heads != 0) return TQ_ERR_INVALID_ARG;
  // more than 16 query heads per kv head: only the matrix-core kernels,
  // which take them in passes (head_dim 128)
  const int G = num_q_heads / g.num_kv_heads;
  if (G > 16 && tq::plan_decode(g, ctx->opts, batch > 0 ? batch : 1, num_q_heads, max_seq_len).mfma == 0)
    return TQ_ERR_UNSUPPORTED;
  if (batch == 0) return TQ_OK;
  if (!q || !cache || !block_table || !seq_lens || !out) return TQ_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_blocks_per_seq) * g.block_size < max_seq_len)
    return TQ_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(cache, 16) || !aligned(out, 16) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4))
    return TQ_ERR_ALIGNMENT;
  tq::DecodePlan plan = tq::plan_decode(g, ctx->opts, batch, num_q_heads, max_seq_len);
  if (plan.workspace_bytes > 0) {
    if (!workspace || workspace_bytes < plan.workspace_bytes) return TQ_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return TQ_ERR_ALIGNMENT;
  }
  tq_status ds = check_device(ctx);
  if (ds != TQ_OK) return ds;
  if (!(sm_scale > 0.0f)) sm_scale = 1.0f / std::sqrt(static_cast<float>(g.head_dim));
  hipError_t e = tq::launch_decode(g, ctx->d_tables, ctx->d_errs, plan, static_cast<const uint16_t*>(q), cache,
                                   num_blocks, block_table, max_blocks_per_seq, seq_lens, batch,
                                   num_q_heads, sm_scale, out, out_is_fp32, workspace,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}
}  // namespace

extern "C" {

tq_status tq_host_codebook(int head_dim, int bits, int codebook_mode, float* centroids_host,
                           float* midpoints_host) {
  if (!centroids_host || !midpoints_host) return TQ_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return TQ_ERR_UNSUPPORTED;
  return host_codebook(head_dim, bits, codebook_mode, centroids_host, midpoints_host);
}

tq_status tq_host_rotation_signs(uint64_t rot_seed, int head_dim, int sign_flip,
                                 int8_t* signs_host) {
  if (!signs_host) return TQ_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return TQ_ERR_UNSUPPORTED;
  rotation_signs(rot_seed, head_dim, sign_flip != 0, signs_host);
  return TQ_OK;
}

tq_status tq_host_haar_matrix(uint64_t rot_seed, int head_dim, float* q_host) {
  if (!q_host) return TQ_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return TQ_ERR_UNSUPPORTED;
  std::vector<float> q32;
  haar_matrix(rot_seed, head_dim, q32);
  std::memcpy(q_host, q32.data(), q32.size() * sizeof(float));
  return TQ_OK;
}

int64_t tq_host_slot_bytes(int preset, int head_dim) {
  if (preset < TQ_K8V4 || preset > TQ_3BIT_NC) return -1;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return -1;
  return slot_bytes_for(preset, head_dim);
}

const char* tq_status_str(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID_ARG: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case TQ_ERR_ALIGNMENT: return "misaligned pointer or stride";
    case TQ_ERR_WORKSPACE: return "workspace too small";
    case TQ_ERR_HIP: return "HIP runtime error";
    case TQ_ERR_NO_DEVICE: return "no gfx950 device";
    default: return "unknown status";
  }
}

tq_status tq_codebook_init(tq_ctx** out, int preset, int head_dim, int num_kv_heads,
                           int block_size, uint64_t rot_seed, int sign_flip, int codebook_mode,
                           void* stream) {
  return tq_codebook_init_layout(out, preset, head_dim, num_kv_heads, block_size, rot_seed,
                                 sign_flip, codebook_mode, TQ_LAYOUT_AOS, stream);
}

int tq_layout_of(const tq_ctx* ctx) { return ctx ? (ctx->geo.soa ? TQ_LAYOUT_SOA : TQ_LAYOUT_AOS) : -1; }

tq_status tq_codebook_init_layout(tq_ctx** out, int preset, int head_dim, int num_kv_heads,
                                  int block_size, uint64_t rot_seed, int sign_flip,
                                  int codebook_mode, int layout, void* stream) {
  if (!out) return TQ_ERR_INVALID_ARG;
  *out = nullptr;
  if (preset < TQ_K8V4 || preset > TQ_3BIT_NC) return TQ_ERR_INVALID_ARG;
  if (layout != TQ_LAYOUT_AOS && layout != TQ_LAYOUT_SOA) return TQ_ERR_INVALID_ARG;
  if (layout == TQ_LAYOUT_SOA && preset == TQ_K8V4) return TQ_ERR_UNSUPPORTED;
  if (codebook_mode != TQ_CODEBOOK_LLOYD_MAX_EXACT && codebook_mode != TQ_CODEBOOK_PAGE_TRAPZ &&
      codebook_mode != TQ_CODEBOOK_BETA_EXACT)
    return TQ_ERR_INVALID_ARG;
  if (num_kv_heads < 1 || num_kv_heads > 64) return TQ_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return TQ_ERR_UNSUPPORTED;
  if (block_size != 16 && block_size != 32 && block_size != 64 && block_size != 128)
    return TQ_ERR_UNSUPPORTED;

  tq_ctx* c = new (std::nothrow) tq_ctx();
  if (!c) return TQ_ERR_INVALID_ARG;
  c->preset = preset;
  c->codebook_mode = codebook_mode;
  Geometry& g = c->geo;
  g.head_dim = head_dim;
  g.num_kv_heads = num_kv_heads;
  g.block_size = block_size;
  g.key_bits = key_bits_of(preset);
  g.value_bits = value_bits_of(preset);
  g.norm_correction = preset == TQ_K8V4 ? 0 : 1;
  g.key_code_bytes = g.key_bits == 8 ? head_dim : (head_dim * g.key_bits + 7) / 8;
  g.key_packed = g.key_bits == 8 ? head_dim : g.key_code_bytes + 2;
  g.value_code_bytes = (head_dim * g.value_bits + 7) / 8;
  g.slot = slot_bytes_for(preset, head_dim);
  g.soa = layout == TQ_LAYOUT_SOA ? 1 : 0;
  // the split page has the slotted page's size: no slot padding to drop
  if (g.soa && g.slot != g.key_packed + g.value_code_bytes + 4) {
    delete c;
    return TQ_ERR_UNSUPPORTED;
  }
  c->r_d = static_cast<float>(1.0 / std::sqrt(static_cast<double>(head_dim)));

  c->levels = 0;
  std::memset(c->centroids, 0, sizeof(c->centroids));
  std::memset(c->midpoints, 0, sizeof(c->midpoints));
  if (g.key_bits != 8) {
    tq_status cs = host_codebook(head_dim, g.key_bits, codebook_mode, c->centroids, c->midpoints);
    if (cs != TQ_OK) {
      delete c;
      return cs;
    }
    c->levels = 1 << g.key_bits;
  }
  // sign_flip: 0 pure Hadamard, TQ_ROTATION_HAAR the Haar matrix, other
  // nonzero values the seeded-sign Hadamard
  g.haar = sign_flip == TQ_ROTATION_HAAR && g.key_bits != 8 ? 1 : 0;
  rotation_signs(rot_seed, head_dim, sign_flip != 0 && !g.haar, c->signs);
  c->d_rot = nullptr;

  DevTables host{};
  std::memcpy(host.centroids, c->centroids, sizeof(host.centroids));
  std::memcpy(host.midpoints, c->midpoints, sizeof(host.midpoints));
  for (int j = 0; j < head_dim; ++j)
    if (c->signs[j] < 0) host.sign_bits[j / 32] |= 1u << (j % 32);
  g.bins_ok = c->levels && build_bins(c->midpoints, c->levels - 1, host);
  if (!g.bins_ok) host.bin_count = 0;

  if (hipGetDevice(&c->device) != hipSuccess) {
    delete c;
    return TQ_ERR_NO_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, c->device) != hipSuccess ||
      std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    delete c;
    return TQ_ERR_NO_DEVICE;
  }
  c->scratch = noalloc_scratch(c->device);
  if (c->scratch == nullptr) {
    delete c;
    return TQ_ERR_HIP;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (g.haar) {
    std::vector<float> q32;
    haar_matrix(rot_seed, head_dim, q32);
    const size_t bytes = q32.size() * sizeof(float);
    if (hipMalloc(&c->d_rot, bytes) != hipSuccess) {
      delete c;
      return TQ_ERR_HIP;
    }
    if (hipMemcpy(c->d_rot, q32.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
      (void)hipFree(c->d_rot);
      delete c;
      return TQ_ERR_HIP;
    }
    host.rot = c->d_rot;
  }
  c->d_errs = nullptr;
  if (hipMalloc(&c->d_tables, sizeof(DevTables)) != hipSuccess) {
    if (c->d_rot) (void)hipFree(c->d_rot);
    delete c;
    return TQ_ERR_HIP;
  }
  const DevErrors no_errors{};
  if (hipMalloc(&c->d_errs, sizeof(DevErrors)) != hipSuccess ||
      hipMemcpyAsync(c->d_tables, &host, sizeof(DevTables), hipMemcpyHostToDevice, st) !=
          hipSuccess ||
      hipMemcpyAsync(c->d_errs, &no_errors, sizeof(DevErrors), hipMemcpyHostToDevice, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess) {
    if (c->d_errs) (void)hipFree(c->d_errs);
    (void)hipFree(c->d_tables);
    if (c->d_rot) (void)hipFree(c->d_rot);
    delete c;
    return TQ_ERR_HIP;
  }
  c->opts = tq_decode_options{};
  *out = c;
  return TQ_OK;
}

tq_status tq_destroy(tq_ctx* ctx) {
  if (!ctx) return TQ_OK;
  tq_status st = TQ_OK;
  if (ctx->d_tables && hipFree(ctx->d_tables) != hipSuccess) st = TQ_ERR_HIP;
  if (ctx->d_errs && hipFree(ctx->d_errs) != hipSuccess) st = TQ_ERR_HIP;
  if (ctx->d_rot && hipFree(ctx->d_rot) != hipSuccess) st = TQ_ERR_HIP;
  delete ctx;
  return st;
}

int64_t tq_slot_bytes(const tq_ctx* ctx) { return ctx ? ctx->geo.slot : -1; }

int64_t tq_cache_bytes(const tq_ctx* ctx, int64_t num_blocks) {
  if (!ctx || num_blocks < 0) return -1;
  return num_blocks * ctx->geo.block_size * ctx->geo.num_kv_heads * ctx->geo.slot;
}

tq_status tq_get_tables(const tq_ctx* ctx, float* centroids_host, float* midpoints_host,
                        int8_t* signs_host) {
  if (!ctx) return TQ_ERR_INVALID_ARG;
  if (centroids_host && ctx->levels)
    std::memcpy(centroids_host, ctx->centroids, sizeof(float) * ctx->levels);
  if (midpoints_host && ctx->levels)
    std::memcpy(midpoints_host, ctx->midpoints, sizeof(float) * (ctx->levels - 1));
  if (signs_host) std::memcpy(signs_host, ctx->signs, ctx->geo.head_dim);
  return TQ_OK;
}

tq_status tq_store(const tq_ctx* ctx, const void* k, const void* v, int64_t kv_token_stride,
                   const int64_t* slot_mapping, int64_t num_tokens, uint8_t* cache,
                   int64_t num_blocks, void* stream) {
  if (!ctx) return TQ_ERR_INVALID_ARG;
  if (num_tokens < 0 || num_blocks < 0) return TQ_ERR_INVALID_ARG;
  if (num_tokens == 0) return TQ_OK;
  if (!k || !v || !slot_mapping || !cache) return TQ_ERR_INVALID_ARG;
  const Geometry& g = ctx->geo;
  if (kv_token_stride < static_cast<int64_t>(g.num_kv_heads) * g.head_dim)
    return TQ_ERR_INVALID_ARG;
  if (kv_token_stride % 8 != 0 || !aligned(k, 16) || !aligned(v, 16) || !aligned(cache, 16) ||
      !aligned(slot_mapping, 8))
    return TQ_ERR_ALIGNMENT;
  tq_status ds = check_device(ctx);
  if (ds != TQ_OK) return ds;
  hipError_t e = tq::launch_store(g, ctx->d_tables, ctx->d_errs, static_cast<const uint16_t*>(k),
                                  static_cast<const uint16_t*>(v), kv_token_stride, slot_mapping,
                                  num_tokens, cache, num_blocks, ctx->r_d,
                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

size_t tq_decode_workspace_bytes(const tq_ctx* ctx, int batch, int num_q_heads,
                                 int max_seq_len) {
  if (!ctx || batch < 0 || num_q_heads <= 0 || max_seq_len < 0) return 0;
  if (num_q_heads % ctx->geo.num_kv_heads != 0) return 0;
  return tq::plan_decode(ctx->geo, ctx->opts, batch, num_q_heads, max_seq_len).workspace_bytes;
}

tq_status tq_decode(const tq_ctx* ctx, const void* q, const uint8_t* cache, int64_t num_blocks,
                    const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                    int batch, int num_q_heads, int max_seq_len, float sm_scale, void* out,
                    int out_is_fp32, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(ctx, q, cache, num_blocks, block_table, max_blocks_per_seq, seq_lens, batch,
                     num_q_heads, max_seq_len, sm_scale, out, out_is_fp32, workspace,
                     workspace_bytes, stream);
}

tq_status tq_decode_noalloc(const tq_ctx* ctx, const void* q, const uint8_t* cache,
                            int64_t num_blocks, const int32_t* block_table, int max_blocks_per_seq,
                            const int32_t* seq_lens, int batch, int num_q_heads, int max_seq_len,
                            float sm_scale, void* out, int out_is_fp32, void* stream) {
  if (!ctx) return TQ_ERR_INVALID_ARG;
  // the scratch array is the workspace: a plan that needs more is refused
  // before anything is enqueued (decode_impl checks the size)
  return decode_impl(ctx, q, cache, num_blocks, block_table, max_blocks_per_seq, seq_lens, batch,
                     num_q_heads, max_seq_len, sm_scale, out, out_is_fp32, ctx->scratch,
                     kNoAllocScratchBytes, stream);
}

size_t tq_decode_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

tq_status tq_dequant(const tq_ctx* ctx, const uint8_t* cache, int64_t num_blocks,
                     const int32_t* block_table_row, int max_blocks, int seq_len, void* k_out,
                     void* v_out, int out_is_fp32, void* stream) {
  if (!ctx) return TQ_ERR_INVALID_ARG;
  const Geometry& g = ctx->geo;
  if (seq_len < 0 || max_blocks < 0 || num_blocks < 0) return TQ_ERR_INVALID_ARG;
  if (seq_len == 0) return TQ_OK;
  if (!cache || !block_table_row || !k_out || !v_out) return TQ_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_blocks) * g.block_size < seq_len) return TQ_ERR_INVALID_ARG;
  if (!aligned(cache, 16) || !aligned(block_table_row, 4) || !aligned(k_out, 16) || !aligned(v_out, 16))
    return TQ_ERR_ALIGNMENT;
  tq_status ds = check_device(ctx);
  if (ds != TQ_OK) return ds;
  hipError_t e = tq::launch_dequant(g, ctx->d_tables, ctx->d_errs, cache, num_blocks, block_table_row, seq_len, k_out,
                                    v_out, out_is_fp32, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

namespace {
// workspace of a continuation: decode workspace, then q_len lengths, then the
// q_len x max_blocks expanded table (each part 256-byte aligned)
struct ContinuationSpace {
  size_t decode, lens_off, table_off, total;
};
ContinuationSpace continuation_space(const Geometry& g, const tq_decode_options& opts, int q_len,
                                     int num_q_heads, int seq_len, int max_blocks) {
  ContinuationSpace c;
  c.decode = tq::plan_decode(g, opts, q_len, num_q_heads, seq_len).workspace_bytes;
  c.lens_off = (c.decode + 255) & ~static_cast<size_t>(255);
  c.table_off = (c.lens_off + 4 * static_cast<size_t>(q_len) + 255) & ~static_cast<size_t>(255);
  c.total = c.table_off + 4 * static_cast<size_t>(q_len) * max_blocks;
  return c;
}
}  // namespace

size_t tq_continuation_workspace_bytes(const tq_ctx* ctx, int q_len, int num_q_heads, int seq_len,
                                       int max_blocks) {
  if (!ctx || q_len <= 0 || num_q_heads <= 0 || seq_len < q_len || max_blocks <= 0) return 0;
  if (num_q_heads % ctx->geo.num_kv_heads != 0) return 0;
  return continuation_space(ctx->geo, ctx->opts, q_len, num_q_heads, seq_len, max_blocks).total;
}

tq_status tq_decode_continuation(const tq_ctx* ctx, const void* q, const uint8_t* cache,
                                 int64_t num_blocks, const int32_t* block_table_row, int max_blocks,
                                 int seq_len, int q_len, int num_q_heads, float sm_scale, void* out,
                                 int out_is_fp32, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (!ctx) return TQ_ERR_INVALID_ARG;
  const Geometry& g = ctx->geo;
  if (q_len <= 0 || seq_len < q_len || max_blocks <= 0 || num_q_heads <= 0 || num_blocks < 0)
    return TQ_ERR_INVALID_ARG;
  if (num_q_heads % g.num_kv_heads != 0) return TQ_ERR_INVALID_ARG;
  if (num_q_heads / g.num_kv_heads > 16 &&
      tq::plan_decode(g, ctx->opts, q_len, num_q_heads, seq_len).mfma == 0)
    return TQ_ERR_UNSUPPORTED;
  if (!q || !cache || !block_table_row || !out || !workspace) return TQ_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_blocks) * g.block_size < seq_len) return TQ_ERR_INVALID_ARG;
  if (!aligned(workspace, 256)) return TQ_ERR_ALIGNMENT;
  if (!aligned(block_table_row, 4)) return TQ_ERR_ALIGNMENT;
  const ContinuationSpace c = continuation_space(g, ctx->opts, q_len, num_q_heads, seq_len, max_blocks);
  if (workspace_bytes < c.total) return TQ_ERR_WORKSPACE;
  tq_status ds = check_device(ctx);
  if (ds != TQ_OK) return ds;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* lens = reinterpret_cast<int32_t*>(ws + c.lens_off);
  int32_t* table = reinterpret_cast<int32_t*>(ws + c.table_off);
  hipError_t e = tq::launch_expand_rows(block_table_row, max_blocks, seq_len - q_len, q_len, lens, table,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return TQ_ERR_HIP;
  return tq_decode(ctx, q, cache, num_blocks, table, max_blocks, lens, q_len, num_q_heads, seq_len, sm_scale,
                   out, out_is_fp32, c.decode > 0 ? workspace : nullptr, c.decode, stream);
}

tq_status tq_get_device_error(const tq_ctx* ctx, int32_t* code_host, int clear, void* stream) {
  if (!ctx || !code_host) return TQ_ERR_INVALID_ARG;
  tq_status ds = check_device(ctx);
  if (ds != TQ_OK) return ds;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // both host buffers live until the stream has synchronised
  DevErrors w{};
  const DevErrors zero{};
  if (hipMemcpyAsync(&w, ctx->d_errs, sizeof(w), hipMemcpyDeviceToHost, st) != hipSuccess)
    return TQ_ERR_HIP;
  if (clear) {
    if (hipMemcpyAsync(ctx->d_errs, &zero, sizeof(zero), hipMemcpyHostToDevice, st) != hipSuccess)
      return TQ_ERR_HIP;
  }
  if (hipStreamSynchronize(st) != hipSuccess) return TQ_ERR_HIP;
  *code_host = (w.slot ? 1 : 0) | (w.page ? 2 : 0) | (w.len ? 4 : 0);
  return TQ_OK;
}

tq_status tq_set_decode_options(tq_ctx* ctx, const tq_decode_options* opts) {
  if (!ctx) return TQ_ERR_INVALID_ARG;
  if (!opts) {
    ctx->opts = tq_decode_options{};
    return TQ_OK;
  }
  if (opts->kernel < TQ_DECODE_KERNEL_AUTO || opts->kernel > TQ_DECODE_KERNEL_GENERAL)
    return TQ_ERR_INVALID_ARG;
  if (opts->ring_waves != 0 && opts->ring_waves != 8 && opts->ring_waves != 16)
    return TQ_ERR_INVALID_ARG;
  if (opts->page_heads != 0 && opts->page_heads != 1 && opts->page_heads != 2 &&
      opts->page_heads != 4)
    return TQ_ERR_INVALID_ARG;
  ctx->opts = *opts;
  ctx->opts.dynamic_claims = opts->dynamic_claims != 0 ? 1 : 0;
  return TQ_OK;
}

tq_status tq_get_decode_options(const tq_ctx* ctx, tq_decode_options* opts) {
  if (!ctx || !opts) return TQ_ERR_INVALID_ARG;
  *opts = ctx->opts;
  return TQ_OK;
}

}  // extern "C"
