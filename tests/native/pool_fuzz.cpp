// Randomized driver of the page allocator (host C++), built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_pool_sanitized.py: admissions over shared prompt
// prefixes, releases, retains, allocations and defragmentations with the jobs' pages remapped,
// then calls with bad arguments, which must be refused. Exit status 0 = no finding.
#include "pkv.h"
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>
int main() {
  std::mt19937 rng(7);
  long ops = 0, fails = 0;
  for (int trial = 0; trial < 40; ++trial) {
    const int P = 4 + (int)(rng() % 60);
    pkv_pool* pool = pkv_pool_create(P);
    if (!pool) return 1;
    std::vector<std::vector<int32_t>> jobs;
    for (int step = 0; step < 400; ++step) {
      const unsigned r = rng() % 100;
      ++ops;
      if (r < 45) {
        // prompts drawn from a few prefixes so pages get reused
        const int n = 1 + (int)(rng() % 1500);
        std::vector<int32_t> toks(n);
        const int fam = (int)(rng() % 3);
        for (int i = 0; i < n; ++i) toks[i] = (i < 600) ? fam * 1000 + i : (int32_t)(rng() % 32000);
        const int cap = (n + 255) / 256;
        std::vector<int32_t> pages(cap);
        int32_t got = 0, cached = 0;
        if (pkv_pool_admit(pool, toks.data(), n, pages.data(), cap, &got, &cached) == PKV_OK) {
          pages.resize(got);
          jobs.push_back(pages);
        } else {
          ++fails;
        }
      } else if (r < 75 && !jobs.empty()) {
        const size_t j = rng() % jobs.size();
        if (pkv_pool_release(pool, jobs[j].data(), (int32_t)jobs[j].size()) != PKV_OK) return 2;
        jobs.erase(jobs.begin() + j);
      } else if (r < 85) {
        const int n = (int)(rng() % 4);
        std::vector<int32_t> pages(n + 1);
        if (pkv_pool_alloc(pool, n, pages.data()) == PKV_OK) {
          pages.resize(n);
          jobs.push_back(pages);
        }
      } else if (r < 90 && !jobs.empty()) {
        const size_t j = rng() % jobs.size();
        if (pkv_pool_retain(pool, jobs[j].data(), (int32_t)jobs[j].size()) != PKV_OK) return 3;
        jobs.push_back(jobs[j]);
      } else {
        std::vector<int32_t> remap(P), src(P), dst(P);
        int32_t moves = 0;
        const int mr = (int)(rng() % 2);
        if (pkv_pool_defrag(pool, mr, remap.data(), src.data(), dst.data(), &moves) != PKV_OK) return 4;
        for (auto& j : jobs)
          for (auto& p : j) p = remap[p];
      }
      int32_t st[4];
      if (pkv_pool_stats(pool, st) != PKV_OK) return 5;
    }
    for (auto& j : jobs) pkv_pool_release(pool, j.data(), (int32_t)j.size());
    pkv_pool_destroy(pool);
  }
  // bad inputs: every call must refuse without touching memory
  pkv_pool* pool = pkv_pool_create(3);
  int32_t bad[2] = {7, -1};
  if (pkv_pool_release(pool, bad, 2) == PKV_OK) return 6;
  if (pkv_pool_retain(pool, bad, 2) == PKV_OK) return 7;
  if (pkv_pool_admit(pool, nullptr, 5, nullptr, 0, nullptr, nullptr) == PKV_OK) return 8;
  pkv_pool_destroy(pool);
  printf("ok: %ld operations, %ld refused admissions\n", ops, fails);
  return 0;
}
