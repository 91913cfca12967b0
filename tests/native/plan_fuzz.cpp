// Random plans through the host planner (fake device addresses), built with the
// address and undefined-behaviour sanitizers by tests/test_planner_sanitized.py: every
// plan must be well formed and every error path clean.
#include <cstdio>
#include <cstdint>
#include <random>
#include <vector>
#include "muon.h"
extern "C" void muon_internal_release(muon_plan*) {}
int main() {
    std::mt19937_64 rng(20261202);
    const int64_t dims[] = {1, 32, 64, 96, 200, 512, 1024, 1100, 2048, 3000, 4096, 8704};
    int ok = 0, too_small = 0;
    for (int trial = 0; trial < 400; ++trial) {
        std::vector<muon_param_desc> d;
        uint64_t addr = 1ull << 40;
        const int nb = 1 + (int)(rng() % 5);
        for (int b = 0; b < nb; ++b) {
            const int64_t r = dims[rng() % 12], c = dims[rng() % 12];
            const int cnt = 1 + (int)(rng() % 150);
            for (int k = 0; k < cnt; ++k) {
                muon_param_desc p{};
                p.ndim = 2; p.rows = r; p.cols = c;
                p.grad_dtype = (rng() & 1) ? MUON_DTYPE_F32 : MUON_DTYPE_BF16;
                p.weight = (float*)addr; addr += ((uint64_t)r * c * 4 + 511) / 256 * 256;
                p.momentum = (float*)addr; addr += ((uint64_t)r * c * 4 + 511) / 256 * 256;
                p.grad = (const void*)addr; addr += ((uint64_t)r * c * 4 + 511) / 256 * 256;
                d.push_back(p);
            }
        }
        for (int pass = 0; pass < 2; ++pass) {
            muon_plan_opts o{};
            o.flags = MUON_PLAN_PIPELINE;
            o.max_workspace_bytes = pass ? (uint64_t)(1 + rng() % 64) << 26 : 0;
            muon_plan* p = nullptr;
            const muon_status st = muon_plan_buckets(d.data(), (int64_t)d.size(), &o, &p);
            if (st == MUON_ERR_WORKSPACE_TOO_SMALL) { ++too_small; continue; }
            if (st != MUON_OK) { std::printf("trial %d: %s\n", trial, muon_last_error()); return 1; }
            uint64_t ws = 0;
            muon_plan_workspace_bytes(p, &ws);
            if (o.max_workspace_bytes && ws > o.max_workspace_bytes) { std::printf("trial %d: ws over cap\n", trial); return 1; }
            int32_t nc = 0; int64_t inc = 0;
            muon_plan_counts(p, &nc, nullptr, &inc, nullptr);
            int64_t sum = 0;
            for (int32_t c = 0; c < nc; ++c) { muon_chunk_info ci; muon_plan_info(p, c, &ci); if (ci.count < 1) return 2; sum += ci.count; }
            if (sum != inc) return 3;
            muon_plan_destroy(p);
            ++ok;
        }
    }
    std::printf("plans ok %d, too small %d\n", ok, too_small);
    return 0;
}
