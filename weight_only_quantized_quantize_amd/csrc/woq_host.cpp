// Host-side preparation of quantised weights: INT8 per-tensor quantisation,
// outlier channel selection and the global permutation, outlier-aware INT4
// encoding and packing, and the canonical <-> device layout transforms.
//
// Everything here is deterministic: each output element is computed by one
// thread from inputs in a fixed order, so results do not depend on the thread
// count.  Rounding is IEEE: fp32 division, nearbyint under the default
// round-to-nearest-even mode, and fp32 -> fp16 conversion through _Float16.
// Build without fast-math.
#include <cfenv>
#include <cmath>
#include <cstring>
#include <numeric>

#include "woq_internal.h"

namespace {

using woq::parallel_for;

inline uint16_t f32_to_f16_bits(float v) {
    _Float16 h = (_Float16)v;  // IEEE round to nearest even
    uint16_t b;
    std::memcpy(&b, &h, 2);
    return b;
}

inline float f16_bits_to_f32(uint16_t b) {
    _Float16 h;
    std::memcpy(&h, &b, 2);
    return (float)h;
}

inline bool f16_finite(uint16_t b) { return (b & 0x7C00u) != 0x7C00u; }

// Nearest integer, ties to even, of an fp32 value (the process keeps the
// default rounding mode; nearbyintf honours it and raises no exception).
inline float rne(float t) { return std::nearbyintf(t); }

// Nibble placement of the INT4O device layout.  Within a 16-byte chunk that
// covers 32 consecutive background channels, channel 16P + t (P = 0, 1;
// t = 0..15) sits in dword 2P + e at nibble position pos:
//   t = 4e + j      (j = 0..3) -> pos {0, 4, 2, 6}[j]   (the unscaled pairs)
//   t = 8 + 4e + j  (j = 0..3) -> pos {1, 5, 3, 7}[j]   (the pairs read x16)
// so that masking a dword with 0x000F000F / 0x00F000F0, before and after a
// shift by 8, yields fp16 pairs of consecutive channels.
struct NibbleSlot {
    int dword;
    int shift;
};
inline NibbleSlot nibble_slot(int c32) {  // c32 = channel within the chunk, 0..31
    static const int lo_pos[4] = {0, 4, 2, 6};
    static const int hi_pos[4] = {1, 5, 3, 7};
    int P = c32 >> 4, t = c32 & 15;
    int e, pos;
    if (t < 8) {
        e = t >> 2;
        pos = lo_pos[t & 3];
    } else {
        e = (t - 8) >> 2;
        pos = hi_pos[(t - 8) & 3];
    }
    return {2 * P + e, 4 * pos};
}

inline int canonical_code(const uint8_t* row, int64_t col) {
    int nib = (row[col >> 1] >> ((col & 1) * 4)) & 0xF;
    return nib >= 8 ? nib - 16 : nib;
}

}  // namespace

namespace woq {

int int4o_geom(int64_t K, int64_t n_out, woq_int4o_geom* g) {
    if (!g || K < 1) return WOQ_EINVAL;
    if (n_out < 0) n_out = (K + 99) / 100;
    if (n_out > K) return WOQ_EINVAL;
    woq_int4o_geom r;
    r.K = K;
    r.n_out = n_out;
    r.K_bg = K - n_out;
    r.G = ceil_div(r.K_bg, 128);
    r.K_pad = 128 * r.G;
    r.G4 = round_up(r.G, 4);
    r.n_out8 = round_up(n_out, 8);
    r.xp_len = 128 * r.G4 + r.n_out8;
    *g = r;
    return WOQ_OK;
}

bool int4o_geom_valid(const woq_int4o_geom* g) {
    if (!g) return false;
    woq_int4o_geom r;
    if (int4o_geom(g->K, g->n_out, &r) != WOQ_OK) return false;
    return std::memcmp(&r, g, sizeof r) == 0;
}

}  // namespace woq

extern "C" {

const char* woq_strerror(int status) {
    switch (status) {
        case WOQ_OK: return "ok";
        case WOQ_EINVAL: return "invalid argument";
        case WOQ_EALIGN: return "misaligned pointer or leading dimension";
        case WOQ_ENOMEM: return "out of memory";
        case WOQ_EHIP: return "HIP runtime error";
        case WOQ_EUNSUPPORTED: return "unsupported request";
        case WOQ_ERANGE: return "value out of range (non-finite weight or fp16 scale overflow)";
        case WOQ_EIO: return "file input/output error";
        case WOQ_EFORMAT: return "not a pool file, or a damaged one";
        default: return "unknown status";
    }
}

int woq_abi_version(void) { return WOQ_ABI_VERSION; }

int woq_int4o_geometry(int64_t K, int64_t n_out, woq_int4o_geom* g) { return woq::int4o_geom(K, n_out, g); }

// ------------------------------------------------------------------ INT8 --

int woq_quantize_int8(const float* W, int64_t N, int64_t K, int8_t* q, float* scale) {
    if (N < 0 || K < 0 || !scale || ((N * K) > 0 && (!W || !q))) return WOQ_EINVAL;
    const int64_t n = N * K;
    // pass 1: max |W| (order-independent) and finiteness
    int nt = woq::num_threads();
    std::vector<float> part_max(nt + 1, 0.0f);
    std::atomic<int> bad{0};
    std::atomic<int> slot{0};
    parallel_for(
        n,
        [&](int64_t lo, int64_t hi) {
            float m = 0.0f;
            bool nf = false;
            for (int64_t i = lo; i < hi; ++i) {
                float a = std::fabs(W[i]);
                if (!std::isfinite(a)) nf = true;
                else if (a > m) m = a;
            }
            if (nf) bad = 1;
            part_max[slot++] = m;
        },
        1 << 16);
    if (bad) return WOQ_ERANGE;
    float m = 0.0f;
    for (float v : part_max) m = std::max(m, v);
    const float s = m / 127.0f;  // fp32 division
    *scale = (s == 0.0f) ? 0.0f : s;
    if (s == 0.0f) {
        if (n) std::memset(q, 0, (size_t)n);
        return WOQ_OK;
    }
    parallel_for(
        n,
        [&](int64_t lo, int64_t hi) {
            for (int64_t i = lo; i < hi; ++i) {
                float r = rne(W[i] / s);
                r = std::min(127.0f, std::max(-127.0f, r));
                q[i] = (int8_t)r;
            }
        },
        1 << 16);
    return WOQ_OK;
}

// ------------------------------------------------------------------ INT4O --

int woq_colabs_accumulate(const float* W, int64_t N, int64_t K, double* colsum) {
    if (N < 0 || K < 1 || !colsum || (N > 0 && !W)) return WOQ_EINVAL;
    parallel_for(
        K,
        [&](int64_t c0, int64_t c1) {
            std::vector<double> acc((size_t)(c1 - c0), 0.0);
            for (int64_t r = 0; r < N; ++r) {
                const float* row = W + r * K;
                for (int64_t j = c0; j < c1; ++j) acc[j - c0] += std::fabs((double)row[j]);
            }
            for (int64_t j = c0; j < c1; ++j) colsum[j] += acc[j - c0];
        },
        64);
    return WOQ_OK;
}

int woq_outlier_select(const double* colsum, const uint16_t* xprof, int64_t T, int64_t K,
                       int64_t n_out, int32_t* perm) {
    if (!colsum || !xprof || !perm || T < 1 || K < 1) return WOQ_EINVAL;
    if (n_out < 0) n_out = (K + 99) / 100;
    if (n_out > K) return WOQ_EINVAL;
    if (K > INT32_MAX) return WOQ_EINVAL;
    std::vector<double> score((size_t)K);
    std::atomic<int> bad{0};
    parallel_for(
        K,
        [&](int64_t c0, int64_t c1) {
            for (int64_t j = c0; j < c1; ++j) {
                double s = 0.0;
                for (int64_t t = 0; t < T; ++t) {
                    uint16_t h = xprof[t * K + j];
                    if (!f16_finite(h)) bad = 1;
                    s += std::fabs((double)f16_bits_to_f32(h));
                }
                score[j] = (s / (double)T) * colsum[j];
                if (!std::isfinite(score[j])) bad = 1;
            }
        },
        64);
    if (bad) return WOQ_ERANGE;
    std::vector<int32_t> idx((size_t)K);
    std::iota(idx.begin(), idx.end(), 0);
    auto better = [&](int32_t a, int32_t b) {
        return score[a] > score[b] || (score[a] == score[b] && a < b);
    };
    if (n_out > 0 && n_out < K) std::nth_element(idx.begin(), idx.begin() + (n_out - 1), idx.end(), better);
    std::vector<char> is_out((size_t)K, 0);
    if (n_out == K) std::fill(is_out.begin(), is_out.end(), 1);
    else {
        // nth_element leaves the n_out best (under the strict order) in front
        for (int64_t i = 0; i < n_out; ++i) is_out[idx[i]] = 1;
    }
    int64_t p = 0;
    for (int64_t j = 0; j < K; ++j)
        if (!is_out[j]) perm[p++] = (int32_t)j;
    for (int64_t j = 0; j < K; ++j)
        if (is_out[j]) perm[p++] = (int32_t)j;
    return WOQ_OK;
}

int woq_outlier_perm_sums(const double* const* parts, int32_t n_parts, int64_t K, const uint16_t* xprof,
                          int64_t T, int64_t n_out, int32_t* perm) {
    if (!parts || n_parts < 1 || K < 1 || !xprof || !perm || T < 1) return WOQ_EINVAL;
    for (int32_t i = 0; i < n_parts; ++i)
        if (!parts[i]) return WOQ_EINVAL;
    // the parts in the order given, channel by channel (the split over
    // threads decides only which thread adds which channels)
    std::vector<double> total((size_t)K, 0.0);
    woq::parallel_for(
        K,
        [&](int64_t c0, int64_t c1) {
            for (int32_t i = 0; i < n_parts; ++i) {
                const double* p = parts[i];
                for (int64_t j = c0; j < c1; ++j) total[j] += p[j];
            }
        },
        256);
    return woq_outlier_select(total.data(), xprof, T, K, n_out, perm);
}

int woq_outlier_perm(const float* const* Ws, const int64_t* Ns, int32_t n_lin, int64_t K, const uint16_t* xprof,
                     int64_t T, int64_t n_out, int32_t* perm) {
    if (!Ws || !Ns || n_lin < 1 || K < 1 || !xprof || !perm || T < 1) return WOQ_EINVAL;
    for (int32_t i = 0; i < n_lin; ++i)
        if (Ns[i] < 0 || (Ns[i] > 0 && !Ws[i])) return WOQ_EINVAL;
    // each linear's column sums from zero, then the same ordered addition as
    // woq_outlier_perm_sums
    std::vector<std::vector<double>> sums((size_t)n_lin);
    std::vector<const double*> parts((size_t)n_lin);
    for (int32_t i = 0; i < n_lin; ++i) {
        sums[i].assign((size_t)K, 0.0);
        const int rc = woq_colabs_accumulate(Ws[i], Ns[i], K, sums[i].data());
        if (rc) return rc;
        parts[i] = sums[i].data();
    }
    return woq_outlier_perm_sums(parts.data(), n_lin, K, xprof, T, n_out, perm);
}

int woq_quantize_int4o(const float* W, int64_t N, int64_t K, const int32_t* perm, int64_t n_out,
                       uint8_t* packed, uint16_t* scales, uint16_t* w_out) {
    woq_int4o_geom g;
    if (woq::int4o_geom(K, n_out, &g) != WOQ_OK) return WOQ_EINVAL;
    if (N < 0 || !perm) return WOQ_EINVAL;
    if (N > 0 && (!W || (g.K_pad && (!packed || !scales)) || (g.n_out && !w_out))) return WOQ_EINVAL;
    {
        std::vector<char> seen((size_t)K, 0);
        for (int64_t k = 0; k < K; ++k) {
            int32_t v = perm[k];
            if (v < 0 || v >= K || seen[v]) return WOQ_EINVAL;
            seen[v] = 1;
        }
    }
    // reject non-finite weights before writing anything
    std::atomic<int> bad{0};
    parallel_for(
        N * K,
        [&](int64_t lo, int64_t hi) {
            for (int64_t i = lo; i < hi; ++i)
                if (!std::isfinite(W[i])) {
                    bad = 1;
                    return;
                }
        },
        1 << 16);
    if (bad) return WOQ_ERANGE;

    const int64_t half = g.K_pad / 2;
    parallel_for(
        N,
        [&](int64_t r0, int64_t r1) {
            std::vector<float> wp((size_t)K);
            std::vector<int8_t> code((size_t)g.K_pad);
            for (int64_t r = r0; r < r1; ++r) {
                const float* row = W + r * K;
                for (int64_t k = 0; k < K; ++k) wp[k] = row[perm[k]];
                for (int64_t i = 0; i < g.n_out; ++i) w_out[r * g.n_out + i] = f32_to_f16_bits(wp[g.K_bg + i]);
                std::fill(code.begin(), code.end(), (int8_t)0);
                for (int64_t gi = 0; gi < g.G; ++gi) {
                    int64_t lo = 128 * gi, hi = std::min<int64_t>(lo + 128, g.K_bg);
                    float m = 0.0f;
                    for (int64_t k = lo; k < hi; ++k) m = std::max(m, std::fabs(wp[k]));
                    uint16_t s16 = f32_to_f16_bits(m / 7.0f);  // fp32 division, then fp16
                    if (!f16_finite(s16)) {
                        bad = 1;
                        return;
                    }
                    scales[r * g.G + gi] = s16;
                    float s = f16_bits_to_f32(s16);
                    if (s == 0.0f) continue;
                    for (int64_t k = lo; k < hi; ++k) {
                        float t = rne(wp[k] / s);
                        t = std::min(7.0f, std::max(-7.0f, t));
                        code[k] = (int8_t)t;
                    }
                }
                uint8_t* out = packed + r * half;
                for (int64_t j = 0; j < half; ++j)
                    out[j] = (uint8_t)((code[2 * j] & 0xF) | ((code[2 * j + 1] & 0xF) << 4));
            }
        },
        1);
    return bad ? WOQ_ERANGE : WOQ_OK;
}

int woq_unpack_int4(const uint8_t* packed, int64_t N, int64_t K_pad, int8_t* q) {
    if (N < 0 || K_pad < 0 || (K_pad & 1) || ((N * K_pad) > 0 && (!packed || !q))) return WOQ_EINVAL;
    const int64_t half = K_pad / 2;
    parallel_for(
        N,
        [&](int64_t r0, int64_t r1) {
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = 0; c < K_pad; ++c) q[r * K_pad + c] = (int8_t)canonical_code(packed + r * half, c);
        },
        16);
    return WOQ_OK;
}

// ---------------------------------------------------------------- layouts --

int64_t woq_int8_dev_bytes(int64_t N, int64_t K) {
    if (N < 0 || K < 1) return -1;
    return woq::round_up(N, 4) * woq::round_up(K, 64);
}

int woq_layout_int8(const int8_t* q, int64_t N, int64_t K, uint8_t* dev) {
    if (N < 0 || K < 1 || !dev || (N > 0 && !q)) return WOQ_EINVAL;
    const int64_t N4 = woq::round_up(N, 4), Kd = woq::round_up(K, 64);
    parallel_for(
        N4,
        [&](int64_t r0, int64_t r1) {
            for (int64_t r = r0; r < r1; ++r) {
                uint8_t* d = dev + r * Kd;
                for (int64_t k = 0; k < Kd; ++k)
                    d[k] = (uint8_t)(((r < N && k < K) ? (int)q[r * K + k] : 0) + 128);
            }
        },
        16);
    return WOQ_OK;
}

int woq_layout_int8_inverse(const uint8_t* dev, int64_t N, int64_t K, int8_t* q) {
    if (N < 0 || K < 1 || !q || (N > 0 && !dev)) return WOQ_EINVAL;
    const int64_t Kd = woq::round_up(K, 64);
    parallel_for(
        N,
        [&](int64_t r0, int64_t r1) {
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t k = 0; k < K; ++k) q[r * K + k] = (int8_t)((int)dev[r * Kd + k] - 128);
        },
        16);
    return WOQ_OK;
}

int woq_int4o_dev_sizes(int64_t N, const woq_int4o_geom* g, int64_t* codes_bytes, int64_t* scales_bytes,
                        int64_t* wout_bytes) {
    if (N < 0 || !woq::int4o_geom_valid(g)) return WOQ_EINVAL;
    const int64_t N16 = woq::round_up(N, 16);
    if (codes_bytes) *codes_bytes = N16 * 64 * g->G4;
    if (scales_bytes) *scales_bytes = N16 * g->G4 * 2;
    if (wout_bytes) *wout_bytes = N16 * g->n_out8 * 2;
    return WOQ_OK;
}

namespace {

// Tile layout offsets (16-row tiles; see woq.h).
inline int64_t code_chunk_offset(int64_t r, int64_t gi, int c, int64_t G4) {
    return (((r >> 4) * G4 + gi) * 4 + c) * 256 + (r & 15) * 16;      // bytes
}
inline int64_t scale_index(int64_t r, int64_t gi, int64_t G4) { return ((r >> 4) * G4 + gi) * 16 + (r & 15); }
inline int64_t wout_index(int64_t r, int64_t i, int64_t no8) {         // fp16 element i of row r
    return (((r >> 4) * no8 + (i >> 3)) * 16 + (r & 15)) * 8 + (i & 7);
}

}  // namespace

int woq_layout_int4o(const uint8_t* packed, const uint16_t* scales, const uint16_t* w_out, int64_t N,
                     const woq_int4o_geom* g, uint8_t* dev_codes, uint16_t* dev_scales, uint16_t* dev_wout) {
    if (N < 0 || !woq::int4o_geom_valid(g)) return WOQ_EINVAL;
    if ((g->G4 && (!dev_codes || !dev_scales)) || (g->n_out8 && !dev_wout)) return WOQ_EINVAL;
    if (N > 0 && ((g->G && (!packed || !scales)) || (g->n_out && !w_out))) return WOQ_EINVAL;
    const int64_t N16 = woq::round_up(N, 16), G = g->G, G4 = g->G4, half = g->K_pad / 2, no8 = g->n_out8 / 8;
    parallel_for(
        N16,
        [&](int64_t r0, int64_t r1) {
            for (int64_t r = r0; r < r1; ++r) {
                const bool real = r < N;
                for (int64_t gi = 0; gi < G4; ++gi) {
                    for (int c = 0; c < 4; ++c) {
                        uint32_t dw[4] = {0, 0, 0, 0};
                        for (int t = 0; t < 32; ++t) {
                            int code = 0;
                            if (real && gi < G) code = canonical_code(packed + r * half, 128 * gi + 32 * c + t);
                            NibbleSlot s = nibble_slot(t);
                            dw[s.dword] |= (uint32_t)(code + 8) << s.shift;
                        }
                        std::memcpy(dev_codes + code_chunk_offset(r, gi, c, G4), dw, 16);   // little-endian dwords
                    }
                    dev_scales[scale_index(r, gi, G4)] = (real && gi < G) ? scales[r * G + gi] : 0;
                }
                for (int64_t i = 0; i < g->n_out8; ++i)
                    dev_wout[wout_index(r, i, no8)] = (real && i < g->n_out) ? w_out[r * g->n_out + i] : 0;
            }
        },
        16);
    return WOQ_OK;
}

int woq_layout_int4o_inverse(const uint8_t* dev_codes, const uint16_t* dev_scales, const uint16_t* dev_wout,
                             int64_t N, const woq_int4o_geom* g, uint8_t* packed, uint16_t* scales,
                             uint16_t* w_out) {
    if (N < 0 || !woq::int4o_geom_valid(g)) return WOQ_EINVAL;
    if (N > 0 && ((g->G && (!dev_codes || !dev_scales || !packed || !scales)) ||
                  (g->n_out && (!dev_wout || !w_out))))
        return WOQ_EINVAL;
    const int64_t G = g->G, G4 = g->G4, half = g->K_pad / 2, no8 = g->n_out8 / 8;
    parallel_for(
        N,
        [&](int64_t r0, int64_t r1) {
            for (int64_t r = r0; r < r1; ++r) {
                uint8_t* out = packed + r * half;     // not read when the space has no background (half = 0)
                if (half) std::memset(out, 0, (size_t)half);
                for (int64_t gi = 0; gi < G; ++gi) {
                    for (int c = 0; c < 4; ++c) {
                        uint32_t dw[4];
                        std::memcpy(dw, dev_codes + code_chunk_offset(r, gi, c, G4), 16);
                        for (int t = 0; t < 32; ++t) {
                            NibbleSlot s = nibble_slot(t);
                            int code = (int)((dw[s.dword] >> s.shift) & 0xF) - 8;
                            int64_t col = 128 * gi + 32 * c + t;
                            out[col >> 1] |= (uint8_t)((code & 0xF) << ((col & 1) * 4));
                        }
                    }
                    scales[r * G + gi] = dev_scales[scale_index(r, gi, G4)];
                }
                for (int64_t i = 0; i < g->n_out; ++i) w_out[r * g->n_out + i] = dev_wout[wout_index(r, i, no8)];
            }
        },
        16);
    return WOQ_OK;
}

int woq_perm_positions(const int32_t* perm, const woq_int4o_geom* g, uint16_t* pos) {
    if (!perm || !pos || !woq::int4o_geom_valid(g)) return WOQ_EINVAL;
    if (g->xp_len > 65535) return WOQ_EUNSUPPORTED;
    const int64_t K = g->K, K8 = woq::round_up(K, 8), bg = 128 * g->G4;
    for (int64_t j = 0; j < K8; ++j) pos[j] = 0xFFFF;
    for (int64_t k = 0; k < K; ++k) {
        const int64_t j = perm[k];
        if (j < 0 || j >= K || pos[j] != 0xFFFF) {
            for (int64_t i = 0; i < K8; ++i) pos[i] = 0xFFFF;
            return WOQ_EINVAL;
        }
        pos[j] = (uint16_t)(k < g->K_bg ? k : bg + (k - g->K_bg));
    }
    return WOQ_OK;
}

}  // extern "C"
