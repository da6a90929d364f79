// Contraction kernels for fp32 storage.
#include "contract.hpp"

namespace convlower {
template void launch_gemm<float>(const conv_desc&, const void*, const void*, const void*, void*, const void*, uint32_t,
                              hipStream_t);

// The contraction of a ConvLSTM step (fp32 NCHW, lowered input in ws, gate
// rows packed in ws): gates -> cell update -> h_t (h_out) and c_t (c_out).
void launch_lstm_gemm(const conv_desc& d, const void* bias, const void* c_prev, void* h_out, void* c_out,
                      const void* ws, hipStream_t st) {
    const char* wsb = static_cast<const char*>(ws);
    GemmArgs g{};
    g.b = wsb + d.off_filter;
    g.bias = bias;
    g.y = h_out;
    g.c_prev = c_prev;
    g.c_out = c_out;
    g.lstm_kh = int32_t(d.p.K / 4);
    g.M = d.M;
    g.K = int32_t(d.p.K);
    g.PQ = int32_t(d.P * d.Q);
    g.Q = int32_t(d.Q);
    g.C = int32_t(d.p.C);
    g.H = int32_t(d.p.H);
    g.W = int32_t(d.p.W);
    g.R = int32_t(d.p.R);
    g.S = int32_t(d.p.S);
    g.sh = d.p.stride_h;
    g.sw = d.p.stride_w;
    g.ph = d.p.pad_h;
    g.pw = d.p.pad_w;
    g.dh = d.p.dil_h;
    g.dw = d.p.dil_w;
    g.a = wsb + d.off_low;
    g.Kc = int32_t(d.Kl);
    g.ldb = int32_t(d.Kl);
    constexpr TileVariant v = kLstmVariant;
    constexpr int BK = v.bk / 2, NT = 64 * v.wgm * v.wgn;
    using B = DmaRows<float, v.bn, BK, false, false, NT>;
    if (d.p.algo == CONV_ALGO_IM2WIN) {
        g.sP = d.W_used * d.RCp;
        g.sN = d.P * g.sP;
        g.sQ = int64_t(d.p.stride_w) * d.RCp;
        g.RCp = int32_t(d.RCp);
        g.sS = int32_t(int64_t(d.p.dil_w) * d.RCp);
        using A = DmaRows<float, v.bm, BK, true, true, NT>;
        launch_dma_core<float, v.bm, v.bn, BK, v.wgm, v.wgn, v.stages, false, false, A, B, 1>(d, g, st);
    } else {
        g.sQ = d.Kl;
        g.sP = d.Q * d.Kl;
        g.sN = d.P * g.sP;
        g.RCp = int32_t(d.Kl);
        g.sS = 0;
        using A = DmaRows<float, v.bm, BK, true, false, NT>;
        launch_dma_core<float, v.bm, v.bn, BK, v.wgm, v.wgn, v.stages, false, false, A, B, 1>(d, g, st);
    }
}

}  // namespace convlower
