// The host's share of a streamed walk: a thread pool and a host int8 matmul for the experts the
// walk hands to the CPU ("#1282 prefill: STRATA_PREFILL_CPU_SHARE=auto hands a small chunk's
// least-routed experts to the idle CPU pool", "What it does").
//
// Arithmetic per routed row, as the layer defines it: the input row is quantised to q8_1 blocks
// (d = amax/127 by IEEE division, q = roundf(v/d), the stored fp16 d and s = fp16(d * sum q) for
// DS4, the fp32 d for D4), then for every weight row and block b the integer dot I_b of the 32
// weight values with the 32 activation values, y_b = dw * dx * I_b (+ mw * sx for Q4_1), summed
// over b; h = silu(g) * u is quantised to q8_1 along F the same way and goes through the down
// matrix.  The integer dots are exact; the fp32 sums run in SIMD lanes (per block 8 partial dots
// of 4 products each, scaled by dw * dx and accumulated per lane, blocks 2i and 2i + 1 in lanes
// 0-7 and 8-15, the lanes added at the end; Q4_1's min term as a separate 8-lane dot of m and s),
// another order than the GPU's, which is why the host's rows are not bit-identical to the GPU's.
//
// The dot products use AVX-512 VNNI (vpdpbusd on 256-bit vectors) where the host has it, else
// AVX2 (vpmaddubsw + vpmaddwd), else scalar code; the choice is made once at run time.  The two
// SIMD paths are one body that differs only in the integer dot (the same sums of 4 byte
// products per lane), so their rows are identical.  (512-bit vectors, two blocks per vpdpbusd,
// measured slower on an AVX-512 Xeon: the lane moves that build the two blocks' operands cost
// more than the halved dot instructions saved.)  Q8_0's signed weights go through the
// sign trick (|w| times x with w's sign) so that the unsigned-by-signed byte products never
// saturate.
#include "cpu_share.hpp"

#include <immintrin.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>

namespace moe {

namespace {

uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

// IEEE binary16 from its definition (1 sign, 5 exponent bits biased by 15, 10 fraction bits),
// exactly: a normal half's fields move into binary32's (exponent rebiased by 127 - 15); a
// subnormal is m * 2^-24 (m < 2^10, so the product is exact).  Called for every weight block's
// scales, so it stays a few integer operations (a libm call per scale dominated small chunks).
inline float half_to_float(uint16_t h) {
  const uint32_t e = (h >> 10) & 31u, m = h & 1023u, sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t bits;
  if (e == 0) {
    const float v = (float)m * 5.9604644775390625e-8f;  // 2^-24
    memcpy(&bits, &v, 4);
  } else if (e == 31) {
    bits = 0x7f800000u | (m << 13);  // infinity, or a NaN keeping its payload
  } else {
    bits = ((e + 112u) << 23) | (m << 13);
  }
  bits |= sign;
  float f;
  memcpy(&f, &bits, 4);
  return f;
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

// A q8_1 row of n values, decoded for the dot products (one contiguous piece of scratch):
//   q   int8 [n]            the block values, block b at 32 b
//   dxe float [n/64][16]    per pair of blocks (2i, 2i + 1): dx of block 2i in 8 lanes, then dx of
//                           block 2i + 1 in 8 lanes (the scale vector the dot products multiply)
//   sx  float [n/32]        s of each block (DS4: fp16(d * sum q) as fp32; D4: 0)
struct QRow {
  const int8_t* q;
  const float* dxe;
  const float* sx;
};
size_t qrow_bytes(int n) { return (size_t)n + (size_t)(n / 64) * 64 + (size_t)(n / 32) * 4; }
QRow qrow_at(uint8_t* base, int n) {
  QRow r;
  r.q = reinterpret_cast<const int8_t*>(base);
  r.dxe = reinterpret_cast<const float*>(base + n);
  r.sx = reinterpret_cast<const float*>(base + n + (size_t)(n / 64) * 64);
  return r;
}

// q8_1 of n values v (n a multiple of 128) into a QRow at base.
void quantize_row(const float* v, int n, bool d4, uint8_t* base) {
  int8_t* q = reinterpret_cast<int8_t*>(base);
  float* dxe = reinterpret_cast<float*>(base + n);
  float* sx = reinterpret_cast<float*>(base + n + (size_t)(n / 64) * 64);
  for (int b = 0; b < n / 32; ++b) {
    const float* x = v + 32 * b;
    float amax = 0.0f;
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(x[j]));
    float dx = 0.0f, s = 0.0f;
    if (amax == 0.0f) {
      memset(q + 32 * b, 0, 32);
    } else {
      const float d = amax / 127.0f;
      int S = 0;
      for (int j = 0; j < 32; ++j) {
        const int qj = (int)roundf(x[j] / d);
        q[32 * b + j] = (int8_t)qj;
        S += qj;
      }
      if (d4) {
        dx = d;
      } else {
        dx = half_to_float(float_to_half(d));
        const float p = d * (float)S;  // rounded to fp32 before the fp16 rounding
        s = half_to_float(float_to_half(p));
      }
    }
    for (int l = 0; l < 8; ++l) dxe[16 * (b >> 1) + 8 * (b & 1) + l] = dx;
    sx[b] = s;
  }
}

// out[r] = sum over the weight row's nblk blocks of y_b for the activation rows xr[r], r < nr.
template <int WT>
void dots_scalar(const uint8_t* wrow, int nblk, const QRow* xr, int nr, float* out) {
  const int bb = WT == 1 ? 20 : 34;
  for (int r = 0; r < nr; ++r) {
    float acc = 0.0f;
    for (int b = 0; b < nblk; ++b) {
      const uint8_t* blk = wrow + (size_t)b * bb;
      const int8_t* x = xr[r].q + 32 * b;
      const float dx = xr[r].dxe[16 * (b >> 1) + 8 * (b & 1)];
      int I = 0;
      if (WT == 1) {
        for (int j = 0; j < 16; ++j) I += (blk[4 + j] & 15) * x[j] + (blk[4 + j] >> 4) * x[j + 16];
        acc += half_to_float(rd16(blk)) * dx * (float)I + half_to_float(rd16(blk + 2)) * xr[r].sx[b];
      } else {
        for (int j = 0; j < 32; ++j) I += (int8_t)blk[2 + j] * x[j];
        acc += half_to_float(rd16(blk)) * dx * (float)I;
      }
    }
    out[r] = acc;
  }
}

// The SIMD paths.  Per pair of blocks and activation row: 16 lanes of 4-product integer dots
// (lanes 0-7 block 2i, 8-15 block 2i + 1, two 8-lane accumulators), converted to fp32, times
// dw * dx (exact for DS4: two fp16 significands), added into the accumulators with one fma.  At
// the end lanes l and l + 8 are added, then the 8 lanes in a fixed tree, then Q4_1's min term,
// itself an 8-lane dot of the weight row's m with the activation row's s.
#define MOE_HSUM8(T, v)                                                                  \
  T __m128 s4_ = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));    \
  const __m128 s2_ = _mm_add_ps(s4_, _mm_movehl_ps(s4_, s4_));                           \
  const float hsum_ = _mm_cvtss_f32(_mm_add_ss(s2_, _mm_shuffle_ps(s2_, s2_, 1)));

template <int WT>
__attribute__((target("avx2,fma"))) inline void unpack_pair_avx2(const uint8_t* blk,
                                                                 __m256i* w0, __m256i* w1) {
  const int bb = WT == 1 ? 20 : 34;
  if (WT == 1) {
    const __m128i mk = _mm_set1_epi8(15);
    const __m128i a = _mm_loadu_si128(reinterpret_cast<const __m128i*>(blk + 4));
    const __m128i b = _mm_loadu_si128(reinterpret_cast<const __m128i*>(blk + bb + 4));
    *w0 = _mm256_set_m128i(_mm_and_si128(_mm_srli_epi16(a, 4), mk), _mm_and_si128(a, mk));
    *w1 = _mm256_set_m128i(_mm_and_si128(_mm_srli_epi16(b, 4), mk), _mm_and_si128(b, mk));
  } else {
    *w0 = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(blk + 2));
    *w1 = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(blk + bb + 2));
  }
}

// Q4_1's min term of one activation row: sum_b m_b * s_b as an 8-lane fp32 dot (the same code
// in both SIMD paths).
__attribute__((target("avx2,fma"))) inline float mterm8(const float* mw, const float* sx,
                                                        int nblk) {
  __m256 a = _mm256_setzero_ps();
  int b = 0;
  for (; b + 8 <= nblk; b += 8)
    a = _mm256_fmadd_ps(_mm256_loadu_ps(mw + b), _mm256_loadu_ps(sx + b), a);
  if (b < nblk) {  // nblk is a multiple of 4: one half-filled step
    const __m256 z = _mm256_setzero_ps();
    a = _mm256_fmadd_ps(_mm256_insertf128_ps(z, _mm_loadu_ps(mw + b), 0),
                        _mm256_insertf128_ps(z, _mm_loadu_ps(sx + b), 0), a);
  }
  MOE_HSUM8(const, a)
  return hsum_;
}

// The SIMD paths, one body for both instruction sets (only the integer dot differs).
#define MOE_SIMD_DOTS(NAME, TARGET, DOT8)                                                       \
  template <int WT>                                                                             \
  __attribute__((target(TARGET))) void NAME(const uint8_t* wrow, int nblk, const QRow* xr,      \
                                            int nr, float* out, float* mw) {                   \
    constexpr int kChunk = 4; /* rows per pass over the weight row (16 accumulators) */         \
    const int bb = WT == 1 ? 20 : 34;                                                           \
    if (WT == 1)                                                                                \
      for (int b = 0; b < nblk; ++b) mw[b] = half_to_float(rd16(wrow + (size_t)b * bb + 2));   \
    for (int r0 = 0; r0 < nr; r0 += kChunk) {                                                   \
      const int m = std::min(kChunk, nr - r0);                                                  \
      __m256 lo[kChunk], hi[kChunk];                                                            \
      for (int i = 0; i < kChunk; ++i) lo[i] = hi[i] = _mm256_setzero_ps();                     \
      for (int b = 0; b < nblk; b += 2) {                                                       \
        const uint8_t* blk = wrow + (size_t)b * bb;                                             \
        __m256i w0, w1;                                                                         \
        unpack_pair_avx2<WT>(blk, &w0, &w1);                                                    \
        const __m256i a0 = WT == 1 ? w0 : _mm256_sign_epi8(w0, w0);                             \
        const __m256i a1 = WT == 1 ? w1 : _mm256_sign_epi8(w1, w1);                             \
        const __m256 d0 = _mm256_set1_ps(half_to_float(rd16(blk)));                             \
        const __m256 d1 = _mm256_set1_ps(half_to_float(rd16(blk + bb)));                        \
        for (int i = 0; i < m; ++i) {                                                           \
          const QRow& x = xr[r0 + i];                                                           \
          __m256i x0 = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(x.q + 32 * b));      \
          __m256i x1 = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(x.q + 32 * b + 32)); \
          if (WT != 1) {                                                                        \
            x0 = _mm256_sign_epi8(x0, w0);                                                      \
            x1 = _mm256_sign_epi8(x1, w1);                                                      \
          }                                                                                     \
          const float* e = x.dxe + 8 * b; /* the pair's 16 lanes */                             \
          lo[i] = _mm256_fmadd_ps(_mm256_cvtepi32_ps(DOT8(a0, x0)),                              \
                                  _mm256_mul_ps(d0, _mm256_loadu_ps(e)), lo[i]);                \
          hi[i] = _mm256_fmadd_ps(_mm256_cvtepi32_ps(DOT8(a1, x1)),                              \
                                  _mm256_mul_ps(d1, _mm256_loadu_ps(e + 8)), hi[i]);            \
        }                                                                                       \
      }                                                                                         \
      for (int i = 0; i < m; ++i) {                                                             \
        const __m256 v = _mm256_add_ps(lo[i], hi[i]);                                           \
        MOE_HSUM8(const, v)                                                                     \
        out[r0 + i] = WT == 1 ? hsum_ + mterm8(mw, xr[r0 + i].sx, nblk) : hsum_;                \
      }                                                                                         \
    }                                                                                           \
  }

#define MOE_DOT8_AVX2(a, x) _mm256_madd_epi16(_mm256_maddubs_epi16(a, x), _mm256_set1_epi16(1))
#define MOE_DOT8_VNNI(a, x) _mm256_dpbusd_epi32(_mm256_setzero_si256(), a, x)
MOE_SIMD_DOTS(dots_avx2, "avx2,fma", MOE_DOT8_AVX2)
MOE_SIMD_DOTS(dots_vnni, "avx2,fma,avx512f,avx512vl,avx512bw,avx512vnni", MOE_DOT8_VNNI)

typedef void (*DotsFn)(const uint8_t*, int, const QRow*, int, float*, float*);

template <int WT>
void dots_scalar_fn(const uint8_t* w, int nblk, const QRow* xr, int nr, float* out, float*) {
  dots_scalar<WT>(w, nblk, xr, nr, out);
}

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
      __builtin_cpu_supports("avx512bw") && __builtin_cpu_supports("avx512f") &&
      __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma"))
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
  if (wt == 1) return i == 2 ? dots_vnni<1> : i == 1 ? dots_avx2<1> : dots_scalar_fn<1>;
  return i == 2 ? dots_vnni<0> : i == 1 ? dots_avx2<0> : dots_scalar_fn<0>;
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
  const size_t xrb = qrow_bytes(H), hrb = qrow_bytes(F);
  sc.act.resize((size_t)n_rows * xrb);
  sc.hq.resize((size_t)n_rows * hrb);
  sc.g.resize((size_t)n_rows * F);
  sc.u.resize((size_t)n_rows * F);
  sc.h.resize((size_t)n_rows * F + (size_t)std::max(nbh, nbf));  // the tail holds m (Q4_1)
  float* mw = sc.h.data() + (size_t)n_rows * F;
  std::vector<QRow> xr(n_rows), hr(n_rows);
  std::vector<float> tmp(n_rows);
  for (int r = 0; r < n_rows; ++r) {
    quantize_row(x_rows[r], H, d4, sc.act.data() + (size_t)r * xrb);
    xr[r] = qrow_at(sc.act.data() + (size_t)r * xrb, H);
    hr[r] = qrow_at(sc.hq.data() + (size_t)r * hrb, F);
  }
  const size_t mat = (size_t)F * nbh * bb;  // bytes of gate (and of up)
  const uint8_t* gate = expert;
  const uint8_t* up = expert + mat;
  const uint8_t* down = expert + 2 * mat;
  for (int n = 0; n < F; ++n) {
    dots(gate + (size_t)n * nbh * bb, nbh, xr.data(), n_rows, tmp.data(), mw);
    for (int r = 0; r < n_rows; ++r) sc.g[(size_t)r * F + n] = tmp[r];
    dots(up + (size_t)n * nbh * bb, nbh, xr.data(), n_rows, tmp.data(), mw);
    for (int r = 0; r < n_rows; ++r) sc.u[(size_t)r * F + n] = tmp[r];
  }
  for (size_t k = 0; k < (size_t)n_rows * F; ++k) {
    const float g = sc.g[k];
    sc.h[k] = g / (1.0f + expf(-g)) * sc.u[k];
  }
  for (int r = 0; r < n_rows; ++r)
    quantize_row(sc.h.data() + (size_t)r * F, F, d4, sc.hq.data() + (size_t)r * hrb);
  for (int i = 0; i < H; ++i) {
    dots(down + (size_t)i * nbf * bb, nbf, hr.data(), n_rows, tmp.data(), mw);
    for (int r = 0; r < n_rows; ++r) out[(size_t)r * H + i] = tmp[r];
  }
}

// ---- the pool -------------------------------------------------------------------------------
CpuPool::CpuPool(int n_threads) {
  try {
    for (int i = 1; i < n_threads; ++i) workers_.emplace_back([this, i] { loop(i); });
  } catch (...) {  // a thread could not start: stop and join the ones that did, then report
    {
      std::lock_guard<std::mutex> lk(mu_);
      stop_ = true;
    }
    go_.notify_all();
    for (std::thread& t : workers_) t.join();
    throw;
  }
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
