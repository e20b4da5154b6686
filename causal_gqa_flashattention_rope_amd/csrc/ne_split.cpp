// ne_split.cpp -- host plan of the key-range split of the longest causal row blocks.
//
// With causal masking, row block rb of a (batch, KV head) group visits about rb + 1 key tiles, so
// when a launch holds only one or two row blocks per CU slot the longest blocks finish last while
// most CUs idle.  The plan cuts the blocks rb >= rs into np pieces of contiguous key tiles and
// orders all jobs longest-first; (rs, np) is the choice whose simulated greedy dispatch (each job
// to the slot that frees first, as the hardware dispatcher does) ends earliest, counting a fixed
// cost per job (operand loads, epilogue) and per piece (writing or reading the partial result).
// Plans are cached per shape: they depend only on the shape, never on the data or the device.
#include <algorithm>
#include <cstdint>
#include <functional>
#include <mutex>
#include <queue>
#include <vector>

#include "ne_launch.hpp"

namespace ne {
namespace {

constexpr int kCus = 256;            // CUs of the chip the plan is made for
constexpr double kJobCost = 1.0;     // per job, in key tiles
// extra per piece of a split block, in key tiles: the hand-off (partial result through memory,
// agent-scope release / acquire, which write back and invalidate the XCD's L2 and so also cost
// the other workgroups there) measured at several tiles' time -- splitting pays only where the
// unsplit order leaves most CUs idle (a group or two per launch), not for a 20% imbalance
constexpr double kPieceCost = 4.0;
constexpr double kMinGain = 0.8;     // split only if the simulated end drops below this fraction

struct Entry {
    int T, G, ngrp, BM, wg, maxp;
    int njobs, rs, np, nrb;
    std::vector<unsigned short> job;
};

double simulate(const std::vector<double>& cost, int ngrp, int slots) {
    std::priority_queue<double, std::vector<double>, std::greater<double>> q;
    for (int i = 0; i < slots; ++i) q.push(0.0);
    double end = 0.0;
    for (double c : cost)
        for (int g = 0; g < ngrp; ++g) {
            const double t = q.top() + c;
            q.pop();
            q.push(t);
            end = std::max(end, t);
        }
    return end;
}

struct Job {
    double cost;
    int rb, piece;
};

// jobs of one group for (rs, np), longest first (ties: later block first, then piece order)
std::vector<Job> jobs_for(const std::vector<int>& tiles, int rs, int np) {
    std::vector<Job> j;
    const int nrb = (int)tiles.size();
    for (int rb = 0; rb < nrb; ++rb) {
        if (rb >= rs) {
            const int n = tiles[rb];
            for (int p = 0; p < np; ++p)
                j.push_back({(double)(n * (p + 1) / np - n * p / np) + kJobCost + kPieceCost, rb, p});
        } else {
            j.push_back({(double)tiles[rb] + kJobCost, rb, 0});
        }
    }
    std::stable_sort(j.begin(), j.end(), [](const Job& a, const Job& b) {
        if (a.cost != b.cost) return a.cost > b.cost;
        if (a.rb != b.rb) return a.rb > b.rb;
        return a.piece < b.piece;
    });
    return j;
}

Entry make_plan(int T, int G, int ngrp, int BM, int wg, int maxp) {
    Entry e{T, G, ngrp, BM, wg, maxp, 0, 0, 1, 0, {}};
    const int64_t TG = (int64_t)T * G;
    const int64_t nrb64 = (TG + BM - 1) / BM;
    e.nrb = (int)std::min<int64_t>(nrb64, INT32_MAX);
    const int slots = kCus * wg;
    // enough blocks per slot, or too many to list: the longest-first order balances by itself
    if (nrb64 > 16383 || (int64_t)ngrp * nrb64 > (int64_t)4 * slots) return e;
    std::vector<int> tiles(e.nrb);
    for (int rb = 0; rb < e.nrb; ++rb)
        tiles[rb] = (int)(std::min<int64_t>((int64_t)rb * BM + BM - 1, TG - 1) / G / 64 + 1);
    std::vector<double> cost;
    auto eval = [&](const std::vector<Job>& j) {
        cost.clear();
        for (const Job& x : j) cost.push_back(x.cost);
        return simulate(cost, ngrp, slots);
    };
    double best = eval(jobs_for(tiles, e.nrb, 1));
    const double base = best;
    int brs = e.nrb, bnp = 1;
    // candidate first split blocks: every block for short lists, else 32 evenly spaced ones
    const int step = std::max(1, e.nrb / 32);
    for (int np = 2; np <= std::min(maxp, 4); ++np)
        for (int rs = e.nrb - 1; rs >= 0; rs -= step) {
            if (tiles[rs] < 2 * np) break;  // tiles grow with rb: smaller rs only shortens pieces
            if ((int64_t)rs + (int64_t)(e.nrb - rs) * np > kMaxSplitJobs) break;
            const double m = eval(jobs_for(tiles, rs, np));
            if (m < best) { best = m; brs = rs; bnp = np; }
        }
    if (bnp == 1 || best > kMinGain * base) return e;  // not worth the hand-off
    const std::vector<Job> j = jobs_for(tiles, brs, bnp);
    e.njobs = (int)j.size();
    e.rs = brs;
    e.np = bnp;
    for (const Job& x : j) e.job.push_back((unsigned short)(x.rb << 2 | x.piece));
    return e;
}

std::mutex g_mu;
std::vector<Entry>* g_cache = nullptr;

}  // namespace

void split_plan(int T, int G, int ngrp, int BM, int wg_per_cu, int max_np, SplitPlan* out) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_cache) g_cache = new std::vector<Entry>();  // kept for the process (entries are small)
    const Entry* hit = nullptr;
    for (const Entry& e : *g_cache)
        if (e.T == T && e.G == G && e.ngrp == ngrp && e.BM == BM && e.wg == wg_per_cu && e.maxp == max_np) hit = &e;
    if (!hit) {
        if (g_cache->size() >= 256) g_cache->erase(g_cache->begin());
        g_cache->push_back(make_plan(T, G, ngrp, BM, wg_per_cu, max_np));
        hit = &g_cache->back();
    }
    out->njobs = hit->njobs;
    out->rs = hit->rs;
    out->np = hit->np;
    out->nrb = hit->nrb;
    std::copy(hit->job.begin(), hit->job.end(), out->job);
}

}  // namespace ne
