// Host anchor sampler (GLM 5.2 DSpark training-design page, §2 "Anchor
// sampling": N anchors drawn at random from the valid positions; a valid A
// lies in [0, S-2] with loss_mask[A] = loss_mask[A+1] = 1, and §6 "eval_mask"
// / appendix A option 2 reset loss_mask[S-1] to 0 on read).
//
// The page leaves the random draw open; this library fixes it as an
// integer-only procedure so that any implementation reproduces it exactly:
// SplitMix64 (Steele, Lea & Flood 2014) drives a partial Fisher-Yates shuffle
// of the ascending candidate list, and the N drawn positions are returned in
// ascending order.
#include <algorithm>
#include <cstring>
#include <vector>

#include "dspark_attn.h"

namespace {

struct SplitMix64 {
    uint64_t state;
    uint64_t next() {
        state += 0x9E3779B97F4A7C15ull;   // golden-ratio Weyl increment
        uint64_t z = state;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
};

}  // namespace

extern "C" dspark_status dspark_select_anchors_host(const uint8_t* loss_mask, int32_t S,
                                                    int32_t num_anchors, uint64_t seed,
                                                    int32_t* anchors, uint8_t* keep) {
    if (S < 1 || num_anchors < 0) return DSPARK_EINVAL;
    if (!loss_mask || (num_anchors > 0 && (!anchors || !keep))) return DSPARK_EINVAL;
    std::vector<int32_t> cand;
    cand.reserve(S);
    for (int32_t a = 0; a + 1 < S; ++a) {
        const bool cur = loss_mask[a] != 0;
        const bool nxt = (a + 1 == S - 1) ? false : (loss_mask[a + 1] != 0);  // lm[S-1] := 0
        if (cur && nxt) cand.push_back(a);
    }
    const size_t n = static_cast<size_t>(num_anchors);
    if (cand.size() <= n) {
        for (size_t i = 0; i < n; ++i) {
            anchors[i] = i < cand.size() ? cand[i] : 0;
            keep[i] = i < cand.size() ? 1 : 0;
        }
        return DSPARK_OK;
    }
    SplitMix64 rng{seed};
    const uint64_t m = cand.size();
    for (uint64_t i = 0; i < n; ++i) {
        const uint64_t j = i + rng.next() % (m - i);
        std::swap(cand[i], cand[j]);
    }
    std::sort(cand.begin(), cand.begin() + n);
    for (size_t i = 0; i < n; ++i) {
        anchors[i] = cand[i];
        keep[i] = 1;
    }
    return DSPARK_OK;
}
