from emulated_fp32_matrix_amd.ceiling import main

main()
