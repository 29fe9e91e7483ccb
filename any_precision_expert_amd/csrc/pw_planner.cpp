// Width planner (PagedWeight pages, "Technical summary: PagedWeight", Core
// components 2: quality-aware runtime planner).  Under a memory target the
// planner greedily takes the width reductions with the lowest damage per
// byte saved; frequently routed ("hot") experts are protected by a higher
// width floor and a damage multiplier.  The pages' damage score also uses an
// offline Hessian-weighted sensitivity and a prompt-specific residual, which
// need trained weights: here the sensitivity is an input and the residual is
// left out.  Pure host code (no device).
#include <algorithm>
#include <cstring>
#include <set>
#include <new>
#include <vector>

#include "../../include/pw.h"
#include "pw_internal.h"

namespace pw {
pw_status plan_fail(const char* msg);
// an exception inside a planner call as a status: OOM for host memory
// exhausted, else INVALID (the entry points return statuses, never exceptions)
pw_status plan_exception(const char* fn, bool oom);
}

namespace {

struct Block {
    int64_t plane_b;  // bytes of one plane: R * K / 8
    int64_t R;
    double weight;    // sensitivity x (routing share + eps) x multiplier
    int floor;
};

// q bit-planes plus LUT_q (R rows of 2^q fp16 entries)
int64_t block_bytes(const Block& b, int q) { return (int64_t)q * b.plane_b + b.R * (2LL << q); }

// damage added by lowering from q to q - 1 (quantisation error power grows
// about 4x per dropped bit: 3 * 4^(8 - q) in units of the 8-bit error)
double drop_damage(const Block& b, int q) { return b.weight * (3.0 * (double)(1LL << (2 * (8 - q)))); }

}  // namespace

template <class F>
pw_status plan_guarded(const char* fn, F&& body)
{
    try {
        return body();
    } catch (const std::bad_alloc&) {
        return pw::plan_exception(fn, true);
    } catch (...) {
        return pw::plan_exception(fn, false);
    }
}

extern "C" pw_status pw_plan_widths(int L, int E, int H, int I, const uint8_t* q_cur, const double* mass,
                                    const float* sens, const pw_plan_params* p, int64_t byte_target, uint8_t* q_out,
                                    int64_t* bytes_out)
{
    return plan_guarded("pw_plan_widths", [&]() -> pw_status {
        using namespace pw;
        if (!q_cur || !mass || !sens || !p || !q_out) return plan_fail("pw_plan_widths: null pointer");
        if (L < 1 || E < 1 || H < 32 || I < 32 || H % 32 || I % 32) return plan_fail("pw_plan_widths: shape out of range");
        if (p->q_min < PW_QMIN || p->q_max > PW_QMAX || p->q_min > p->q_max || p->hot_floor > p->q_max)
            return plan_fail("pw_plan_widths: widths out of range");
        const int n = 2 * L * E;
        std::vector<Block> bl(n);
        std::vector<int> q(n);
        for (int l = 0; l < L; ++l) {
            double sum = 0.0;
            for (int e = 0; e < E; ++e) sum += mass[(size_t)l * E + e];
            for (int e = 0; e < E; ++e) {
                const double share = sum > 0.0 ? mass[(size_t)l * E + e] / sum : 0.0;
                const bool hot = p->hot_share > 0.0 && share >= p->hot_share;
                for (int m = 0; m < 2; ++m) {
                    const int b = (l * E + e) * 2 + m;
                    const int R = m == 0 ? 2 * I : H, K = m == 0 ? H : I;
                    Block& x = bl[b];
                    x.plane_b = (int64_t)R * K / 8;
                    x.R = R;
                    x.weight = (double)sens[b] * (share + p->mass_eps) * (hot ? p->hot_mult : 1.0);
                    x.floor = hot ? std::max(p->q_min, p->hot_floor) : p->q_min;
                    q[b] = std::min(std::max((int)q_cur[b], x.floor), p->q_max);
                }
            }
        }
        int64_t total = 0;
        for (int b = 0; b < n; ++b) total += block_bytes(bl[b], q[b]);
        if (total > byte_target) {
            // lower: smallest damage per byte saved first (ties: lower block index)
            std::set<std::pair<double, int>> cand;
            auto key = [&](int b) {
                return drop_damage(bl[b], q[b]) / (double)(block_bytes(bl[b], q[b]) - block_bytes(bl[b], q[b] - 1));
            };
            for (int b = 0; b < n; ++b)
                if (q[b] > bl[b].floor) cand.insert({key(b), b});
            while (total > byte_target && !cand.empty()) {
                const int b = cand.begin()->second;
                cand.erase(cand.begin());
                total -= block_bytes(bl[b], q[b]) - block_bytes(bl[b], q[b] - 1);
                --q[b];
                if (q[b] > bl[b].floor) cand.insert({key(b), b});
            }
        } else {
            // raise: largest damage removed per byte added first, while the target allows
            // (ties: lower block index)
            std::set<std::pair<double, int>> cand;  // (-key, b)
            auto key = [&](int b) {
                return drop_damage(bl[b], q[b] + 1) / (double)(block_bytes(bl[b], q[b] + 1) - block_bytes(bl[b], q[b]));
            };
            for (int b = 0; b < n; ++b)
                if (q[b] < p->q_max) cand.insert({-key(b), b});
            for (;;) {
                auto it = cand.begin();
                for (; it != cand.end(); ++it) {
                    const int b = it->second;
                    if (total + block_bytes(bl[b], q[b] + 1) - block_bytes(bl[b], q[b]) <= byte_target) break;
                }
                if (it == cand.end()) break;
                const int b = it->second;
                cand.erase(it);
                total += block_bytes(bl[b], q[b] + 1) - block_bytes(bl[b], q[b]);
                ++q[b];
                if (q[b] < p->q_max) cand.insert({-key(b), b});
            }
        }
        for (int b = 0; b < n; ++b) q_out[b] = (uint8_t)q[b];
        if (bytes_out) *bytes_out = total;
        return PW_OK;
    });
}

// One commit event of the fixed-fraction schedule: among the routed blocks
// not skipped and not at the bound (q > 3 when lowering, q < 8 when
// raising), the n_change with the least routing mass of their expert (both
// modules of an expert share it; ties: lower block id) move one bit.
extern "C" pw_status pw_plan_event(int L, int E, const uint8_t* q_cur, const double* mass, const uint8_t* skip,
                                   int lower, int n_change, int32_t* ids_out, uint8_t* q_out, int* n_out)
{
    return plan_guarded("pw_plan_event", [&]() -> pw_status {
        using namespace pw;
        if (!q_cur || !mass || !n_out || (n_change > 0 && (!ids_out || !q_out)))
            return plan_fail("pw_plan_event: null pointer");
        if (L < 1 || E < 1 || n_change < 0) return plan_fail("pw_plan_event: size out of range");
        struct Cand {
            double m;
            int32_t id;
            int b;
        };
        std::vector<Cand> cand;
        for (int l = 0; l < L; ++l)
            for (int e = 0; e < E; ++e)
                for (int m = 0; m < 2; ++m) {
                    const int b = (l * E + e) * 2 + m;
                    const int q = q_cur[b];
                    if (q < PW_QMIN || q > PW_QMAX) return plan_fail("pw_plan_event: width out of range");
                    if ((skip && skip[b]) || (lower ? q <= PW_QMIN : q >= PW_QMAX)) continue;
                    cand.push_back({mass[(size_t)l * E + e], (l * (E + 1) + e) * 2 + m, b});
                }
        std::sort(cand.begin(), cand.end(), [](const Cand& x, const Cand& y) {
            return x.m < y.m || (x.m == y.m && x.id < y.id);
        });
        const int n = std::min<int>(n_change, (int)cand.size());
        for (int i = 0; i < n; ++i) {
            ids_out[i] = cand[i].id;
            q_out[i] = (uint8_t)(q_cur[cand[i].b] + (lower ? -1 : 1));
        }
        *n_out = n;
        return PW_OK;
    });
}
