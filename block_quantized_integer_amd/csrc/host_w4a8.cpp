// host_w4a8.cpp -- the grouped W4A8 GEMM on the host CPU with integer SIMD:
// "A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU"
// (gist.science summary) decodes on the CPU from RAM with a hand-written
// W4A8 kernel built on SSSE3 pmaddubsw (Method 1; Contributions, the
// integer-SIMD decode path).  This is that path for the host CPUs next to an
// MI355X: the same instruction widened to AVX2 (vpmaddubsw, 32 unsigned x
// signed byte products summed in pairs per instruction).
//
// pmaddubsw multiplies unsigned by signed bytes, so the 4-bit codes c (0..15)
// are used as they are and the offset is applied afterwards:
//   P = sum_i (c_i - 8) a_i = sum_i c_i a_i - 8 * sum_i a_i,
// exact in int32 (pair sums are at most 2 * 15 * 128, far from the int16
// limit).  The per-block activation sums are formed once per token.  Each
// block's term P * (da * dw) (the fp16 x fp16 product is exact in fp32) is
// accumulated with one fma, so the result obeys the library's bound
// (nb + 1) * 2^-24 * sum |terms|.  Work is split over threads by routed row
// and column range; results do not depend on the thread count.
#include <immintrin.h>
#include <stdint.h>
#include <string.h>

#include <unistd.h>

#include <algorithm>
#include <cmath>
#include <condition_variable>
#include <mutex>
#include <thread>
#include <vector>

#include "bqi.h"

namespace {

// fp16 bit pattern -> fp32 (exact, subnormals kept), written out so that the
// host path needs no F16C
float h2f(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1f, m = h & 0x3ff;
  uint32_t bits;
  if (e == 0) {
    if (m == 0) {
      bits = sign;
    } else {  // subnormal: m * 2^-24, exactly
      float f = (float)m * 5.9604644775390625e-08f;
      memcpy(&bits, &f, 4);
      bits |= sign;
    }
  } else if (e == 31) {
    bits = sign | 0x7f800000u | (m << 13);
  } else {
    bits = sign | ((e + 112) << 23) | (m << 13);
  }
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

// sum of the eight int32 lanes
__attribute__((target("avx2"))) inline int32_t hsum8(__m256i v) {
  __m128i s = _mm_add_epi32(_mm256_castsi256_si128(v), _mm256_extracti128_si256(v, 1));
  s = _mm_add_epi32(s, _mm_shuffle_epi32(s, 0x4e));
  s = _mm_add_epi32(s, _mm_shuffle_epi32(s, 0xb1));
  return _mm_cvtsi128_si32(s);
}

struct Job {
  const int8_t *aq;
  const uint16_t *ad;
  const int32_t *ids;
  int64_t top_k;
  const uint8_t *wq4;
  const uint16_t *wd;
  int64_t E, n, k;
  float *y;
  const int32_t *asum;  // [n_tokens][k/32] per-block activation sums
  int64_t item0, item1;  // work items = routed row * column chunks
  int64_t col_chunk;
};

__attribute__((target("avx2,fma"))) void run(const Job &J) {
  const int64_t nb = J.k / 32;
  const int64_t chunks = (J.n + J.col_chunk - 1) / J.col_chunk;
  const __m256i lo_mask = _mm256_set1_epi8(0x0f);
  const __m256i ones16 = _mm256_set1_epi16(1);
  for (int64_t it = J.item0; it < J.item1; ++it) {
    const int64_t r = it / chunks, ch = it - r * chunks;
    const int64_t c_begin = ch * J.col_chunk, c_end = std::min(J.n, c_begin + J.col_chunk);
    const int32_t e = J.ids[r];
    float *yr = J.y + r * J.n;
    if (e < 0 || e >= J.E) {
      for (int64_t c = c_begin; c < c_end; ++c) yr[c] = 0.0f;
      continue;
    }
    const int64_t t = r / J.top_k;
    const int8_t *a = J.aq + t * J.k;
    const int32_t *sa = J.asum + t * nb;
    for (int64_t c = c_begin; c < c_end; ++c) {
      const uint8_t *w = J.wq4 + ((int64_t)e * J.n + c) * (J.k / 2);
      const uint16_t *ws = J.wd + ((int64_t)e * J.n + c) * nb;
      float acc = 0.0f;
      for (int64_t b = 0; b < nb; ++b) {
        // 16 packed bytes -> the block's 32 codes in element order: low
        // nibbles are elements 0..15, high nibbles 16..31
        const __m128i p = _mm_loadu_si128(reinterpret_cast<const __m128i *>(w + 16 * b));
        const __m256i pp = _mm256_set_m128i(_mm_srli_epi16(p, 4), p);
        const __m256i codes = _mm256_and_si256(pp, lo_mask);
        const __m256i act = _mm256_loadu_si256(reinterpret_cast<const __m256i *>(a + 32 * b));
        const __m256i pairs = _mm256_maddubs_epi16(codes, act);     // u8 x s8, pairs summed
        const __m256i quads = _mm256_madd_epi16(pairs, ones16);      // -> int32
        const int32_t P = hsum8(quads) - 8 * sa[b];
        const float s = h2f(J.ad[t * nb + b]) * h2f(ws[b]);         // exact
        acc = std::fma((float)P, s, acc);
      }
      yr[c] = acc;
    }
  }
}

// Worker threads kept across calls: starting them anew in every call cost
// about as much as a one-token decode step's work.  The pool starts on first
// use and grows to the largest thread count asked for; one call at a time
// uses it (concurrent callers wait on `call`), and the calling thread runs
// job 0 itself.  Workers wait for a new generation, run their job if the
// call has one for them, and count down `pending`.  The pool is never torn
// down (its threads end with the process); a child made by fork() builds its
// own, since the parent's workers do not exist there.
struct Pool {
  std::mutex call;
  std::mutex m;
  std::condition_variable go, done;
  std::vector<std::thread> workers;
  const Job *jobs = nullptr;
  int n_jobs = 0, pending = 0;
  uint64_t gen = 0;
  pid_t pid = getpid();

  void work(int i) {  // worker i runs job i (i >= 1)
    uint64_t seen = 0;
    for (;;) {
      const Job *job = nullptr;
      {
        std::unique_lock<std::mutex> l(m);
        go.wait(l, [&] { return gen != seen; });
        seen = gen;
        if (i < n_jobs) job = &jobs[i];
      }
      if (!job) continue;
      run(*job);
      std::lock_guard<std::mutex> l(m);
      if (--pending == 0) done.notify_one();
    }
  }

  // Runs jobs 0 .. n-1; jobs that no worker can take (a thread could not be
  // started) run on the calling thread after job 0.
  void run_all(const Job *js, int n) {
    std::lock_guard<std::mutex> c(call);
    try {
      while ((int)workers.size() < n - 1) {
        const int i = (int)workers.size() + 1;
        workers.emplace_back([this, i] { work(i); });
      }
    } catch (...) {
      // no more threads: the calling thread takes the rest
    }
    const int shared = std::min(n, (int)workers.size() + 1);
    {
      std::lock_guard<std::mutex> l(m);
      jobs = js;
      n_jobs = shared;
      pending = shared - 1;
      ++gen;
    }
    go.notify_all();
    run(js[0]);
    for (int i = shared; i < n; ++i) run(js[i]);
    std::unique_lock<std::mutex> l(m);
    done.wait(l, [&] { return pending == 0; });
    jobs = nullptr;
  }
};

Pool *pool_for_this_process() {
  static std::mutex guard;
  static Pool *pool = nullptr;
  std::lock_guard<std::mutex> l(guard);
  if (!pool || pool->pid != getpid()) pool = new Pool;  // (a forked child's copy is left alone)
  return pool;
}

}  // namespace

extern "C" {

BQI_API int qgemm_w4a8_grouped_host(const int8_t *aq, const uint16_t *ad,
                                    int64_t n_tokens, const int32_t *topk_ids,
                                    int64_t top_k, const uint8_t *wq4,
                                    const uint16_t *wd, int64_t n_experts,
                                    int64_t n, int64_t k, float *y,
                                    int nthreads) {
  if (n_tokens < 0 || top_k < 0 || n_experts < 0 || n < 0 || k < 0 || k % 32 != 0)
    return BQI_ESHAPE;
  const int64_t R = n_tokens * top_k;
  if (R == 0 || n == 0) return BQI_OK;
  if (!y || !topk_ids) return BQI_EINVAL;
  if (k > 0 && (!aq || !ad)) return BQI_EINVAL;
  if (k > 0 && n_experts > 0 && (!wq4 || !wd)) return BQI_EINVAL;
  if (!__builtin_cpu_supports("avx2") || !__builtin_cpu_supports("fma"))
    return BQI_ENOTSUP;
  const int64_t nb = k / 32;
  // per-block activation sums, for the offset of the unsigned codes
  std::vector<int32_t> asum((size_t)(n_tokens * nb));
  for (int64_t t = 0; t < n_tokens; ++t)
    for (int64_t b = 0; b < nb; ++b) {
      int32_t s = 0;
      for (int i = 0; i < 32; ++i) s += aq[t * k + 32 * b + i];
      asum[(size_t)(t * nb + b)] = s;
    }
  if (nthreads <= 0) nthreads = (int)std::max(1u, std::thread::hardware_concurrency());
  const int64_t col_chunk = 64;
  const int64_t items = R * ((n + col_chunk - 1) / col_chunk);
  if (nthreads > items) nthreads = (int)items;
  std::vector<Job> jobs((size_t)nthreads);
  for (int i = 0; i < nthreads; ++i)
    jobs[(size_t)i] = Job{aq, ad, topk_ids, top_k, wq4, wd, n_experts, n, k, y,
                          asum.data(), items * i / nthreads, items * (i + 1) / nthreads,
                          col_chunk};
  if (nthreads == 1)
    run(jobs[0]);
  else
    pool_for_this_process()->run_all(jobs.data(), nthreads);
  return BQI_OK;
}

}  // extern "C"
