"""MI355X-native NVFP4 skinny GEMM: Y[M,N] = X[M,K] . dequant(W)[K,N] for M = 1 .. 128."""
