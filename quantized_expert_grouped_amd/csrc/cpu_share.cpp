// The host's share of a streamed walk: a thread pool and a host int8 matmul for the experts the
// walk hands to the CPU ("#1282 prefill: STRATA_PREFILL_CPU_SHARE=auto hands a small chunk's
// least-routed experts to the idle CPU pool", "What it does").
//
// Arithmetic per routed row, as the layer defines it: the input row is quantised to q8_1 blocks
// (d = amax/127 by IEEE division, q = roundf(v/d), the stored fp16 d and s = fp16(d * sum q) for
// DS4, the fp32 d for D4), then for every weight row and block b the integer dot I_b of the 32
// weight values with the 32 activation values, y_b = dw * dx * I_b (+ mw * sx for Q4_1), summed
// over b; h = silu(g) * u is quantised to q8_1 along F the same way and goes through the down
// matrix.  The integer dots are exact; the fp32 sums run in SIMD lanes (8 partial dots of 4
// products each, scaled and accumulated per lane, then added across lanes), another order than
// the GPU's, which is why the host's rows are not bit-identical to the GPU's.
//
// The dot products use AVX-512 VNNI (vpdpbusd on 256-bit vectors) where the host has it, else
// AVX2 (vpmaddubsw + vpmaddwd), else scalar code; the choice is made once at run time.  Q8_0's
// signed weights go through the usual sign trick (|w| times x with w's sign) so that the
// unsigned-by-signed byte products never saturate.
#include "cpu_share.hpp"

#include <immintrin.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>

namespace moe {

namespace {

struct ABlk {   // one 32-value block of a q8_1 row, decoded
  int8_t q[32];
  float d;      // the scale as the layer stores it (fp16 -> fp32 exactly for DS4, fp32 for D4)
  float s;      // DS4: fp16(d * sum q) as fp32 (Q4_1's min term); D4: 0
};

uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

// IEEE binary16 from its definition (1 sign, 5 exponent bits biased by 15, 10 fraction bits).
float half_to_float(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  float v;
  if (e == 0)
    v = ldexpf((float)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexpf((float)(1024 + m), e - 25);
  return (h & 0x8000) ? -v : v;
}

// fp32 -> binary16, round to nearest even, subnormals kept, 65520 and above to infinity.
uint16_t float_to_half(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u, ax = x & 0x7fffffffu;
  if (ax >= 0x7f800000u) return (uint16_t)(sign | (ax > 0x7f800000u ? 0x7e00u : 0x7c00u));
  if (ax >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);  // |f| >= 65520
  if (ax < 0x38800000u) {                                     // below 2^-14: a subnormal half
    float a;
    memcpy(&a, &ax, 4);
    return (uint16_t)(sign | (uint32_t)rintf(a * 16777216.0f));  // units of 2^-24, exact scale
  }
  uint32_t half = ((((ax >> 23) - 112u) << 10) | ((ax & 0x7fffffu) >> 13));
  const uint32_t rem = ax & 0x1fffu;
  if (rem > 0x1000u || (rem == 0x1000u && (half & 1u))) ++half;  // a carry moves the exponent
  return (uint16_t)(sign | half);
}

void quantize_row(const float* v, int n, bool d4, ABlk* out) {
  for (int b = 0; b < n / 32; ++b) {
    const float* x = v + 32 * b;
    ABlk& o = out[b];
    float amax = 0.0f;
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(x[j]));
    if (amax == 0.0f) {
      memset(o.q, 0, 32);
      o.d = o.s = 0.0f;
      continue;
    }
    const float d = amax / 127.0f;
    int S = 0;
    for (int j = 0; j < 32; ++j) {
      const int q = (int)roundf(x[j] / d);
      o.q[j] = (int8_t)q;
      S += q;
    }
    if (d4) {
      o.d = d;
      o.s = 0.0f;
    } else {
      o.d = half_to_float(float_to_half(d));
      const float p = d * (float)S;  // rounded to fp32 before the fp16 rounding
      o.s = half_to_float(float_to_half(p));
    }
  }
}

constexpr int kChunk = 8;  // activation rows per pass over a weight row

// out[r] = sum over the row's nblk blocks of y_b for activation rows xr[r], r < nr.
template <int WT>
void dots_scalar(const uint8_t* wrow, int nblk, const ABlk* const* xr, int nr, float* out) {
  const int bb = WT == 1 ? 20 : 34;
  for (int r = 0; r < nr; ++r) {
    float acc = 0.0f;
    for (int b = 0; b < nblk; ++b) {
      const uint8_t* blk = wrow + (size_t)b * bb;
      const ABlk& a = xr[r][b];
      int I = 0;
      if (WT == 1) {
        for (int j = 0; j < 16; ++j)
          I += (blk[4 + j] & 15) * a.q[j] + (blk[4 + j] >> 4) * a.q[j + 16];
        acc += half_to_float(rd16(blk)) * a.d * (float)I + half_to_float(rd16(blk + 2)) * a.s;
      } else {
        for (int j = 0; j < 32; ++j) I += (int8_t)blk[2 + j] * a.q[j];
        acc += half_to_float(rd16(blk)) * a.d * (float)I;
      }
    }
    out[r] = acc;
  }
}

// The SIMD form of dots_scalar, per activation row 8 lanes of partial dots (4 byte products
// each); two copies, one per instruction set, so that the AVX2 one never uses AVX-512.
#define MOE_SIMD_DOTS(NAME, TARGET, DOT8)                                                      \
  template <int WT>                                                                            \
  __attribute__((target(TARGET))) void NAME(const uint8_t* wrow, int nblk,                      \
                                            const ABlk* const* xr, int nr, float* out) {        \
    const int bb = WT == 1 ? 20 : 34;                                                          \
    for (int r0 = 0; r0 < nr; r0 += kChunk) {                                                  \
      const int m = std::min(kChunk, nr - r0);                                                 \
      __m256 acc[kChunk];                                                                      \
      float macc[kChunk];                                                                      \
      for (int i = 0; i < kChunk; ++i) {                                                       \
        acc[i] = _mm256_setzero_ps();                                                          \
        macc[i] = 0.0f;                                                                        \
      }                                                                                        \
      for (int b = 0; b < nblk; ++b) {                                                         \
        const uint8_t* blk = wrow + (size_t)b * bb;                                            \
        __m256i w;                                                                             \
        if (WT == 1) {                                                                         \
          const __m128i qs = _mm_loadu_si128(reinterpret_cast<const __m128i*>(blk + 4));       \
          const __m128i mk = _mm_set1_epi8(15);                                                \
          w = _mm256_set_m128i(_mm_and_si128(_mm_srli_epi16(qs, 4), mk),                       \
                               _mm_and_si128(qs, mk));                                         \
        } else {                                                                               \
          w = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(blk + 2));                   \
        }                                                                                      \
        const __m256i aw = WT == 1 ? w : _mm256_sign_epi8(w, w);                               \
        const float dw = half_to_float(rd16(blk));                                             \
        const float mw = WT == 1 ? half_to_float(rd16(blk + 2)) : 0.0f;                        \
        for (int i = 0; i < m; ++i) {                                                          \
          const ABlk& a = xr[r0 + i][b];                                                       \
          __m256i x = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(a.q));               \
          if (WT != 1) x = _mm256_sign_epi8(x, w);                                             \
          const __m256i p = DOT8(aw, x);                                                       \
          acc[i] = _mm256_fmadd_ps(_mm256_cvtepi32_ps(p), _mm256_set1_ps(dw * a.d), acc[i]);   \
          if (WT == 1) macc[i] += mw * a.s;                                                    \
        }                                                                                      \
      }                                                                                        \
      for (int i = 0; i < m; ++i) {                                                            \
        const __m128 s4 =                                                                      \
            _mm_add_ps(_mm256_castps256_ps128(acc[i]), _mm256_extractf128_ps(acc[i], 1));      \
        const __m128 s2 = _mm_add_ps(s4, _mm_movehl_ps(s4, s4));                               \
        const __m128 s1 = _mm_add_ss(s2, _mm_shuffle_ps(s2, s2, 1));                           \
        out[r0 + i] = _mm_cvtss_f32(s1) + macc[i];                                             \
      }                                                                                        \
    }                                                                                          \
  }

#define MOE_DOT8_AVX2(aw, x) _mm256_madd_epi16(_mm256_maddubs_epi16(aw, x), _mm256_set1_epi16(1))
#define MOE_DOT8_VNNI(aw, x) _mm256_dpbusd_epi32(_mm256_setzero_si256(), aw, x)
MOE_SIMD_DOTS(dots_avx2, "avx2,fma", MOE_DOT8_AVX2)
MOE_SIMD_DOTS(dots_vnni, "avx2,fma,avx512f,avx512vl,avx512bw,avx512vnni", MOE_DOT8_VNNI)

typedef void (*DotsFn)(const uint8_t*, int, const ABlk* const*, int, float*);

int detect_isa_host();

int detect_isa() {
  __builtin_cpu_init();
  // MOE_CPU_ISA=scalar|avx2 caps the choice (to exercise every path on one host)
  const char* cap = getenv("MOE_CPU_ISA");
  const int limit = !cap ? 2 : strcmp(cap, "scalar") == 0 ? 0 : strcmp(cap, "avx2") == 0 ? 1 : 2;
  const int best = detect_isa_host();
  return best < limit ? best : limit;
}

int detect_isa_host() {
  if (__builtin_cpu_supports("avx512vnni") && __builtin_cpu_supports("avx512vl") &&
      __builtin_cpu_supports("avx512bw") && __builtin_cpu_supports("avx2") &&
      __builtin_cpu_supports("fma"))
    return 2;
  if (__builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma")) return 1;
  return 0;
}

int isa() {
  static const int v = detect_isa();
  return v;
}

DotsFn dots_for(int wt) {
  const int i = isa();
  if (wt == 1) return i == 2 ? dots_vnni<1> : i == 1 ? dots_avx2<1> : dots_scalar<1>;
  return i == 2 ? dots_vnni<0> : i == 1 ? dots_avx2<0> : dots_scalar<0>;
}

}  // namespace

const char* cpu_share_isa() {
  const int i = isa();
  return i == 2 ? "avx512-vnni" : i == 1 ? "avx2" : "scalar";
}

void cpu_expert_rows(int wtype, int H, int F, const uint8_t* expert, const float* const* x_rows,
                     int n_rows, float* out, CpuScratch& sc) {
  if (n_rows <= 0) return;
  const int wt = wtype == 1 ? 1 : 0;
  const bool d4 = wtype == 2;
  const int bb = wt == 1 ? 20 : 34;
  const int nbh = H / 32, nbf = F / 32;
  const DotsFn dots = dots_for(wt);
  sc.act.resize((size_t)n_rows * nbh * sizeof(ABlk));
  sc.hq.resize((size_t)n_rows * nbf * sizeof(ABlk));
  sc.g.resize((size_t)n_rows * F);
  sc.u.resize((size_t)n_rows * F);
  sc.h.resize((size_t)n_rows * F);
  ABlk* act = reinterpret_cast<ABlk*>(sc.act.data());
  ABlk* hq = reinterpret_cast<ABlk*>(sc.hq.data());
  std::vector<const ABlk*> xr(n_rows), hr(n_rows);
  std::vector<float> tmp(n_rows);
  for (int r = 0; r < n_rows; ++r) {
    quantize_row(x_rows[r], H, d4, act + (size_t)r * nbh);
    xr[r] = act + (size_t)r * nbh;
    hr[r] = hq + (size_t)r * nbf;
  }
  const size_t mat = (size_t)F * nbh * bb;  // bytes of gate (and of up)
  const uint8_t* gate = expert;
  const uint8_t* up = expert + mat;
  const uint8_t* down = expert + 2 * mat;
  for (int n = 0; n < F; ++n) {
    dots(gate + (size_t)n * nbh * bb, nbh, xr.data(), n_rows, tmp.data());
    for (int r = 0; r < n_rows; ++r) sc.g[(size_t)r * F + n] = tmp[r];
    dots(up + (size_t)n * nbh * bb, nbh, xr.data(), n_rows, tmp.data());
    for (int r = 0; r < n_rows; ++r) sc.u[(size_t)r * F + n] = tmp[r];
  }
  for (size_t k = 0; k < (size_t)n_rows * F; ++k) {
    const float g = sc.g[k];
    sc.h[k] = g / (1.0f + expf(-g)) * sc.u[k];
  }
  for (int r = 0; r < n_rows; ++r) quantize_row(sc.h.data() + (size_t)r * F, F, d4, hq + (size_t)r * nbf);
  for (int i = 0; i < H; ++i) {
    dots(down + (size_t)i * nbf * bb, nbf, hr.data(), n_rows, tmp.data());
    for (int r = 0; r < n_rows; ++r) out[(size_t)r * H + i] = tmp[r];
  }
}

// ---- the pool -------------------------------------------------------------------------------
CpuPool::CpuPool(int n_threads) {
  for (int i = 1; i < n_threads; ++i) workers_.emplace_back([this, i] { loop(i); });
}

CpuPool::~CpuPool() {
  {
    std::lock_guard<std::mutex> lk(mu_);
    stop_ = true;
  }
  go_.notify_all();
  for (std::thread& t : workers_) t.join();
}

void CpuPool::work(int worker) {
  for (;;) {
    const int j = next_.fetch_add(1);
    if (j >= n_jobs_) return;
    fn_(j, worker);
  }
}

void CpuPool::loop(int worker) {
  uint64_t seen = 0;
  for (;;) {
    {
      std::unique_lock<std::mutex> lk(mu_);
      go_.wait(lk, [&] { return stop_ || generation_ != seen; });
      if (stop_) return;
      seen = generation_;
    }
    work(worker);
    {
      std::lock_guard<std::mutex> lk(mu_);
      if (--busy_ == 0) done_.notify_all();
    }
  }
}

void CpuPool::start(int n_jobs, std::function<void(int, int)> fn) {
  {
    std::lock_guard<std::mutex> lk(mu_);
    fn_ = std::move(fn);
    n_jobs_ = n_jobs;
    next_ = 0;
    busy_ = (int)workers_.size();
    ++generation_;
  }
  go_.notify_all();
}

void CpuPool::wait() {
  work(0);
  std::unique_lock<std::mutex> lk(mu_);
  done_.wait(lk, [&] { return busy_ == 0; });
  fn_ = nullptr;
}

}  // namespace moe
