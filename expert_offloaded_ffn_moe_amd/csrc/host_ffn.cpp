// Host (CPU) computation of expert FFNs on the library's internal 4-bit layout
// (see host_ffn.h). Built with AVX-512 code generation enabled for this file
// only; the library calls into it only when host_ffn_supported().
#include "host_ffn.h"

#include <immintrin.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <mutex>
#include <thread>
#include <vector>

namespace moe {

bool host_ffn_supported() {
  __builtin_cpu_init();
  return __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
         __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("f16c");
}

// ----------------------------------------------------------------------------- pool

// Items are handed out through one atomic counter. A worker takes the run's item
// count and function under the lock when it wakes, and a new run starts only when no
// worker is still inside the previous one, so no item of a run is taken twice or
// handed to a worker that holds another run's state.
struct HostPool::Impl {
  std::vector<std::thread> workers;
  std::mutex mu;
  std::condition_variable cv_work, cv_done;
  const std::function<void(int)>* fn = nullptr;
  int n = 0;
  std::atomic<int> next{0};
  int done = 0;           // items finished in the current run
  int active = 0;         // workers inside a run
  unsigned long gen = 0;  // run generation, bumped per run
  bool stop = false;

  int drain(const std::function<void(int)>* f, int nn) {
    int finished = 0;
    for (int i = next.fetch_add(1); i < nn; i = next.fetch_add(1)) {
      (*f)(i);
      ++finished;
    }
    return finished;
  }

  void worker() {
    unsigned long seen = 0;
    for (;;) {
      const std::function<void(int)>* f;
      int nn;
      {
        std::unique_lock<std::mutex> lock(mu);
        cv_work.wait(lock, [&] { return stop || gen != seen; });
        if (stop) return;
        seen = gen;
        f = fn;
        nn = n;
        ++active;
      }
      const int finished = f ? drain(f, nn) : 0;
      {
        std::lock_guard<std::mutex> lock(mu);
        done += finished;
        --active;
      }
      cv_done.notify_all();
    }
  }
};

HostPool::HostPool(int threads) : impl_(new Impl) {
  for (int i = 1; i < std::max(1, threads); ++i) impl_->workers.emplace_back([this] { impl_->worker(); });
}

HostPool::~HostPool() {
  {
    std::lock_guard<std::mutex> lock(impl_->mu);
    impl_->stop = true;
  }
  impl_->cv_work.notify_all();
  for (auto& t : impl_->workers) t.join();
  delete impl_;
}

int HostPool::threads() const { return (int)impl_->workers.size() + 1; }

void HostPool::run(int n, const std::function<void(int)>& fn) {
  if (n <= 0) return;
  Impl* q = impl_;
  {
    std::unique_lock<std::mutex> lock(q->mu);
    q->cv_done.wait(lock, [&] { return q->active == 0; });
    q->fn = &fn;
    q->n = n;
    q->done = 0;
    q->next.store(0);
    ++q->gen;
  }
  q->cv_work.notify_all();
  const int mine = q->drain(&fn, n);
  std::unique_lock<std::mutex> lock(q->mu);
  q->done += mine;
  q->cv_done.wait(lock, [&] { return q->done == q->n && q->active == 0; });
  q->fn = nullptr;
}

// ----------------------------------------------------------------------------- kernels

namespace {

constexpr int kMT = 8;  // tokens per pass over a row block

// The 16 lane words of lanes 16*lq .. 16*lq+15 of one 1 KiB code block, as four
// vectors D[d] = dword d of each lane (lane order).
inline void load_dwords(const uint8_t* blk, __m512i D[4]) {
  const __m512i z0 = _mm512_loadu_si512(blk), z1 = _mm512_loadu_si512(blk + 64);
  const __m512i z2 = _mm512_loadu_si512(blk + 128), z3 = _mm512_loadu_si512(blk + 192);
  // (dwords 0 and 1 of lanes 0-7), (dwords 2 and 3 of lanes 0-7), the same for lanes 8-15
  const __m512i ia = _mm512_setr_epi32(0, 4, 8, 12, 16, 20, 24, 28, 1, 5, 9, 13, 17, 21, 25, 29);
  const __m512i ib = _mm512_setr_epi32(2, 6, 10, 14, 18, 22, 26, 30, 3, 7, 11, 15, 19, 23, 27, 31);
  const __m512i t0 = _mm512_permutex2var_epi32(z0, ia, z1), t1 = _mm512_permutex2var_epi32(z0, ib, z1);
  const __m512i t2 = _mm512_permutex2var_epi32(z2, ia, z3), t3 = _mm512_permutex2var_epi32(z2, ib, z3);
  const __m512i lo = _mm512_setr_epi32(0, 1, 2, 3, 4, 5, 6, 7, 16, 17, 18, 19, 20, 21, 22, 23);
  const __m512i hi = _mm512_setr_epi32(8, 9, 10, 11, 12, 13, 14, 15, 24, 25, 26, 27, 28, 29, 30, 31);
  D[0] = _mm512_permutex2var_epi32(t0, lo, t2);
  D[1] = _mm512_permutex2var_epi32(t0, hi, t2);
  D[2] = _mm512_permutex2var_epi32(t1, lo, t3);
  D[3] = _mm512_permutex2var_epi32(t1, hi, t3);
}

// sum over K of q * s * x_m for 16 rows (lanes 16*lq .. 16*lq+15 of one tile) and
// mc <= kMT token rows x[m] (K fp32 each); xs[m][g]: sum of x[m] over group g.
// Codes are stored as n = q + 8, so sum q x = sum n x - 8 sum x per group.
void rows16(const uint8_t* codes, const uint8_t* scales, int chunks, int groups, int lq, const float* const* x,
            const float* const* xs, int mc, __m512* out) {
  const int cpg = chunks / groups;
  __m512 acc[kMT];
  for (int m = 0; m < kMT; ++m) acc[m] = _mm512_setzero_ps();
  const __m512i mask = _mm512_set1_epi32(0xF);
  for (int g = 0; g < groups; ++g) {
    __m512 accg[kMT];
    for (int m = 0; m < kMT; ++m) accg[m] = _mm512_setzero_ps();
    for (int cc = 0; cc < cpg; ++cc) {
      const int c = g * cpg + cc;
      __m512i D[4];
      load_dwords(codes + (size_t)c * 1024 + lq * 256, D);
      for (int d = 0; d < 4; ++d) {
        for (int j = 0; j < 4; ++j) {
          const __m512 ne = _mm512_cvtepi32_ps(_mm512_and_si512(_mm512_srli_epi32(D[d], 4 * j), mask));
          const __m512 no = _mm512_cvtepi32_ps(_mm512_and_si512(_mm512_srli_epi32(D[d], 16 + 4 * j), mask));
          const int k = 32 * c + 8 * d + 2 * j;
          for (int m = 0; m < mc; ++m) {
            accg[m] = _mm512_fmadd_ps(ne, _mm512_set1_ps(x[m][k]), accg[m]);
            accg[m] = _mm512_fmadd_ps(no, _mm512_set1_ps(x[m][k + 1]), accg[m]);
          }
        }
      }
    }
    const __m512 s = _mm512_cvtph_ps(_mm256_loadu_si256(reinterpret_cast<const __m256i*>(scales + ((size_t)g * 64 + lq * 16) * 2)));
    for (int m = 0; m < mc; ++m) {
      const __m512 t = _mm512_fnmadd_ps(_mm512_set1_ps(8.f), _mm512_set1_ps(xs[m][g]), accg[m]);
      acc[m] = _mm512_fmadd_ps(s, t, acc[m]);
    }
  }
  for (int m = 0; m < mc; ++m) out[m] = acc[m];
}

// float -> bf16 (round to nearest even) -> float, 16 at a time
inline __m512 round_bf16(__m512 v) {
  __m512i u = _mm512_castps_si512(v);
  const __m512i lsb = _mm512_and_si512(_mm512_srli_epi32(u, 16), _mm512_set1_epi32(1));
  u = _mm512_add_epi32(u, _mm512_add_epi32(_mm512_set1_epi32(0x7FFF), lsb));
  u = _mm512_and_si512(u, _mm512_set1_epi32((int)0xFFFF0000u));
  return _mm512_castsi512_ps(u);
}

inline void group_sums(const float* v, int K, int G, float* out) {
  for (int g = 0; g < K / G; ++g) {
    float s = 0.f;
    for (int i = 0; i < G; ++i) s += v[g * G + i];
    out[g] = s;
  }
}

struct Job {
  const uint8_t* blob;
  int M;
  bool h_bf16;
  const float* x;  // [M][H]
  float* h;        // [M][I]
  float* o;        // [M][H]
};

// Gate/up tile t (32 gate + 32 up rows) of one expert for all its tokens: h rows.
void gateup_tile(const Layout& L, const Job& jb, int t, const float* xsum /*[M][H/G]*/) {
  const uint8_t* codes = jb.blob + L.off_gu_codes + (size_t)t * L.gu_chunks * 1024;
  const uint8_t* scales = jb.blob + L.off_gu_scales + (size_t)t * L.gu_groups * 128;
  for (int m0 = 0; m0 < jb.M; m0 += kMT) {
    const int mc = std::min(kMT, jb.M - m0);
    const float* x[kMT];
    const float* xs[kMT];
    for (int m = 0; m < kMT; ++m) {
      const int mm = m0 + std::min(m, mc - 1);
      x[m] = jb.x + (size_t)mm * L.H;
      xs[m] = xsum + (size_t)mm * L.gu_groups;
    }
    __m512 r[4][kMT];  // gate rows 0-15, 16-31, up rows 0-15, 16-31
    for (int lq = 0; lq < 4; ++lq) rows16(codes, scales, (int)L.gu_chunks, (int)L.gu_groups, lq, x, xs, mc, r[lq]);
    for (int m = 0; m < mc; ++m)
      for (int half = 0; half < 2; ++half) {
        alignas(64) float g[16], u[16], hv[16];
        _mm512_store_ps(g, r[half][m]);
        _mm512_store_ps(u, r[2 + half][m]);
        for (int i = 0; i < 16; ++i) hv[i] = g[i] / (1.f + std::exp(-g[i])) * u[i];
        const __m512 hz = _mm512_load_ps(hv);
        _mm512_storeu_ps(jb.h + (size_t)(m0 + m) * L.I + 32 * t + 16 * half, jb.h_bf16 ? round_bf16(hz) : hz);
      }
  }
}

// Down tile t (64 rows of H) of one expert for all its tokens: o rows.
void down_tile(const Layout& L, const Job& jb, int t, const float* hsum /*[M][I/G]*/) {
  const uint8_t* codes = jb.blob + L.off_dn_codes + (size_t)t * L.dn_chunks * 1024;
  const uint8_t* scales = jb.blob + L.off_dn_scales + (size_t)t * L.dn_groups * 128;
  for (int m0 = 0; m0 < jb.M; m0 += kMT) {
    const int mc = std::min(kMT, jb.M - m0);
    const float* x[kMT];
    const float* xs[kMT];
    for (int m = 0; m < kMT; ++m) {
      const int mm = m0 + std::min(m, mc - 1);
      x[m] = jb.h + (size_t)mm * L.I;
      xs[m] = hsum + (size_t)mm * L.dn_groups;
    }
    __m512 r[kMT];
    for (int lq = 0; lq < 4; ++lq) {
      rows16(codes, scales, (int)L.dn_chunks, (int)L.dn_groups, lq, x, xs, mc, r);
      for (int m = 0; m < mc; ++m) _mm512_storeu_ps(jb.o + (size_t)(m0 + m) * L.H + 64 * t + 16 * lq, r[m]);
    }
  }
}

}  // namespace

void host_experts_ffn(const Layout& L, int n_experts, const uint8_t* const* blob, const int* M, const int* x_off,
                      const float* x, float* h, float* o, bool h_bf16, HostPool& pool) {
  if (n_experts <= 0) return;
  std::vector<Job> jobs(n_experts);
  int rows = 0;
  for (int i = 0; i < n_experts; ++i) {
    jobs[i] = Job{blob[i], M[i], h_bf16, x + (size_t)x_off[i] * L.H, h + (size_t)x_off[i] * L.I,
                  o + (size_t)x_off[i] * L.H};
    rows = std::max(rows, x_off[i] + M[i]);
  }
  // group sums of the jobs' token rows of x and (after gate/up) of h
  std::vector<float> xsum((size_t)rows * L.gu_groups), hsum((size_t)rows * L.dn_groups);
  for (int i = 0; i < n_experts; ++i)
    for (int r = x_off[i]; r < x_off[i] + M[i]; ++r)
      group_sums(x + (size_t)r * L.H, (int)L.H, (int)L.G, &xsum[(size_t)r * L.gu_groups]);
  const int gt = (int)L.gu_tiles, dt = (int)L.dn_tiles;
  pool.run(n_experts * gt, [&](int item) {
    const int e = item / gt;
    gateup_tile(L, jobs[e], item % gt, &xsum[(size_t)x_off[e] * L.gu_groups]);
  });
  for (int i = 0; i < n_experts; ++i)
    for (int r = x_off[i]; r < x_off[i] + M[i]; ++r)
      group_sums(h + (size_t)r * L.I, (int)L.I, (int)L.G, &hsum[(size_t)r * L.dn_groups]);
  pool.run(n_experts * dt, [&](int item) {
    const int e = item / dt;
    down_tile(L, jobs[e], item % dt, &hsum[(size_t)x_off[e] * L.dn_groups]);
  });
}

void host_expert_ffn(const Layout& L, const uint8_t* blob, const float* x, int M, float* h, float* o, bool h_bf16,
                     HostPool& pool) {
  const int zero = 0;
  host_experts_ffn(L, 1, &blob, &M, &zero, x, h, o, h_bf16, pool);
}

}  // namespace moe
